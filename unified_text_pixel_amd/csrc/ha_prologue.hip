// Fused q/k RMSNorm + rotary embedding, bound by HBM bandwidth.
//
// Per head row x of length D (hidream-o1-p100a model card, "q/k RMSNorm" and "3-axis
// interleaved mRoPE [24,20,20]"; HunyuanImage 3.0 digest, "Generalized 2D Rotary
// Position Embedding"):
//   y = x / sqrt(mean(x^2) + eps) * w                         (when weights are given)
//   (y[i], y[i+D/2]) <- rotation of the pair by pos[axis(i)] * theta^(-2i/D)
// Every head of a token shares the token's angles, so one workgroup handles one token:
// it gathers the token's D/2 (cos, sin) pairs from the table into LDS once, then D/16
// threads per head row each own 8 pairs, i.e. elements [8c, 8c+8) and [D/2+8c, D/2+8c+8),
// which are 16-byte (bf16) loads and stores. The row's mean square is reduced across
// those D/16 lanes. fp32 math throughout; bf16 results are rounded to nearest even.
#include <algorithm>

#include "ha_internal.h"

namespace ha {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <bool F32>
__device__ inline void load8(const void* base, int64_t off, float* x) {
  if constexpr (F32) {
    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + off);
    f32x4 a = p[0], b = p[1];
    for (int e = 0; e < 4; ++e) { x[e] = a[e]; x[4 + e] = b[e]; }
  } else {
    bf16x8 v = *reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(base) + off);
    for (int e = 0; e < 8; ++e) x[e] = static_cast<float>(v[e]);
  }
}

template <bool F32>
__device__ inline void store8(void* base, int64_t off, const float* x) {
  if constexpr (F32) {
    f32x4* p = reinterpret_cast<f32x4*>(static_cast<float*>(base) + off);
    p[0] = f32x4{x[0], x[1], x[2], x[3]};
    p[1] = f32x4{x[4], x[5], x[6], x[7]};
  } else {
    bf16x8 v;
    for (int e = 0; e < 8; ++e) v[e] = static_cast<__bf16>(x[e]);
    *reinterpret_cast<bf16x8*>(static_cast<__bf16*>(base) + off) = v;
  }
}

template <int D, bool F32>
__global__ __launch_bounds__(1024) void prologue_kernel(PrologueArgs a) {
  constexpr int HALF = D / 2;
  constexpr int TPR = D / 16;  // threads per head row
  __shared__ float2 cs[HALF];
  // token b * S + s, s in [token_begin, S)
  const int run = a.S - a.token_begin;
  const int64_t token = (int64_t)(blockIdx.x / run) * a.S + a.token_begin + blockIdx.x % run;

  if (a.rotate) {
    for (int t = threadIdx.x; t < HALF; t += blockDim.x) {
      int p = a.positions[token * a.n_axes + a.axis[t]];
      p = min(max(p, 0), a.n_pos - 1);
      cs[t] = reinterpret_cast<const float2*>(a.cos_sin)[(int64_t)p * HALF + t];
    }
  }
  __syncthreads();

  const int row = threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  if (row >= a.Hq + a.Hkv) return;  // whole rows drop out together
  const bool isq = row < a.Hq;
  const int h = isq ? row : row - a.Hq;
  const int64_t base = (token * (isq ? a.Hq : a.Hkv) + h) * D;
  const void* in = isq ? a.q_in : a.k_in;
  void* out = isq ? a.q_out : a.k_out;
  const float* w = isq ? a.wq : a.wk;

  float x1[8], x2[8];
  load8<F32>(in, base + 8 * c, x1);
  load8<F32>(in, base + HALF + 8 * c, x2);

  if (w) {
    float ss = 0.f;
    for (int e = 0; e < 8; ++e) ss += x1[e] * x1[e] + x2[e] * x2[e];
    for (int o = 1; o < TPR; o <<= 1) ss += __shfl_xor(ss, o);
    const float inv = 1.0f / sqrtf(ss / (float)D + a.eps);
    for (int e = 0; e < 8; ++e) {
      x1[e] = x1[e] * inv * w[8 * c + e];
      x2[e] = x2[e] * inv * w[HALF + 8 * c + e];
    }
  }
  if (a.rotate) {
    for (int e = 0; e < 8; ++e) {
      const float2 t = cs[8 * c + e];
      const float y1 = x1[e] * t.x - x2[e] * t.y;
      const float y2 = x2[e] * t.x + x1[e] * t.y;
      x1[e] = y1;
      x2[e] = y2;
    }
  }
  if (isq && a.q_scale != 1.f) {
    for (int e = 0; e < 8; ++e) {
      x1[e] *= a.q_scale;
      x2[e] *= a.q_scale;
    }
  }
  store8<F32>(out, base + 8 * c, x1);
  store8<F32>(out, base + HALF + 8 * c, x2);
}

template <int D, bool F32>
hipError_t launch(const PrologueArgs& a, hipStream_t stream) {
  const int threads = ((a.Hq + a.Hkv) * (D / 16) + 63) / 64 * 64;
  hipLaunchKernelGGL((prologue_kernel<D, F32>), dim3((unsigned)((int64_t)a.B * (a.S - a.token_begin))),
                     dim3(threads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prologue(const PrologueArgs& a, hipStream_t stream) {
  if (a.D == 128) return a.f32 ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
  return a.f32 ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
}

}  // namespace ha

// ---------------------------------------------------------------- backward
//
// Gradient of the prologue's inputs from the gradient of its outputs (fp32, before any
// q prescale). Per head row, with g the output gradient:
//   rotary:  the pair rotation is orthogonal, so its input gradient is g rotated by minus
//            the angle: (g1 c + g2 s, g2 c - g1 s)
//   RMSNorm: y = x r w, r = (mean(x^2) + eps)^(-1/2); with u = dy * w,
//            dx = r u - x r^3 mean(x u),  and the weight gradient collects dy * x r
// One workgroup per token, D/16 threads per head row as in the forward; the token's weight
// gradient (its heads' terms staged in LDS and summed in head order) goes to one row of a
// per-token partial array, which launch_dw_reduce then sums over tokens.
namespace ha {
namespace {

template <int D, bool F32>
__global__ __launch_bounds__(1024) void prologue_bwd_kernel(PrologueBwdArgs a) {
  constexpr int HALF = D / 2;
  constexpr int TPR = D / 16;
  __shared__ float2 cs[HALF];
  // this token's dy * x * r per head row, [Hq + Hkv][D] (sized at launch, none without
  // RMSNorm: a small footprint keeps many tokens' loads in flight per CU)
  extern __shared__ float contrib[];
  const int64_t token = blockIdx.x;

  if (a.rotate) {
    for (int t = threadIdx.x; t < HALF; t += blockDim.x) {
      int p = a.positions[token * a.n_axes + a.axis[t]];
      p = min(max(p, 0), a.n_pos - 1);
      cs[t] = reinterpret_cast<const float2*>(a.cos_sin)[(int64_t)p * HALF + t];
    }
  }
  __syncthreads();

  const int row = threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  if (row < a.Hq + a.Hkv) {
    const bool isq = row < a.Hq;
    const int h = isq ? row : row - a.Hq;
    const int64_t base = (token * (isq ? a.Hq : a.Hkv) + h) * D;
    const float* gin = (isq ? a.dq_rot : a.dk_rot) + base;
    const float* w = isq ? a.wq : a.wk;

    float g1[8], g2[8];
    load8<true>(gin, 8 * c, g1);
    load8<true>(gin, HALF + 8 * c, g2);
    if (a.rotate) {
      for (int e = 0; e < 8; ++e) {
        const float2 t = cs[8 * c + e];
        const float y1 = g1[e] * t.x + g2[e] * t.y;
        const float y2 = g2[e] * t.x - g1[e] * t.y;
        g1[e] = y1;
        g2[e] = y2;
      }
    }
    if (w) {
      float x1[8], x2[8];
      load8<F32>(isq ? a.q_in : a.k_in, base + 8 * c, x1);
      load8<F32>(isq ? a.q_in : a.k_in, base + HALF + 8 * c, x2);
      float ss = 0.f, xu = 0.f;
      for (int e = 0; e < 8; ++e) {
        ss += x1[e] * x1[e] + x2[e] * x2[e];
        xu += x1[e] * g1[e] * w[8 * c + e] + x2[e] * g2[e] * w[HALF + 8 * c + e];
      }
      for (int o = 1; o < TPR; o <<= 1) {
        ss += __shfl_xor(ss, o);
        xu += __shfl_xor(xu, o);
      }
      const float r = 1.0f / sqrtf(ss / (float)D + a.eps);
      const float k3 = r * r * r * xu / (float)D;
      for (int e = 0; e < 8; ++e) {
        if (a.dwq_part) {
          contrib[row * D + 8 * c + e] = g1[e] * x1[e] * r;
          contrib[row * D + HALF + 8 * c + e] = g2[e] * x2[e] * r;
        }
        g1[e] = r * g1[e] * w[8 * c + e] - x1[e] * k3;
        g2[e] = r * g2[e] * w[HALF + 8 * c + e] - x2[e] * k3;
      }
    }
    void* out = isq ? a.dq : a.dk;
    store8<F32>(out, base + 8 * c, g1);
    store8<F32>(out, base + HALF + 8 * c, g2);
  }
  if (a.dwq_part) {
    // the token's weight gradients: sums over its q heads and over its k heads, in order
    __syncthreads();
    for (int t = threadIdx.x; t < 2 * D; t += blockDim.x) {
      const int d = t % D;
      const bool q = t < D;
      float s = 0.f;
      for (int r = q ? 0 : a.Hq, e = q ? a.Hq : a.Hq + a.Hkv; r < e; ++r) s += contrib[r * D + d];
      (q ? a.dwq_part : a.dwk_part)[token * D + d] = s;
    }
  }
}

// dw[d] = sum over n rows of part[row][d], in two passes of fixed order: kDwBlocks
// workgroups each sum a contiguous chunk of rows into out[block][d], then one workgroup
// sums those. 1024 threads: 1024 / D threads per column, strided over the chunk. The q and
// k weights go together (blockIdx.y selects the pair of arrays).
constexpr int kDwBlocks = 256;

__global__ __launch_bounds__(1024) void dw_sum_kernel(const float* part_q, const float* part_k, int64_t n, int D,
                                                      float* out_q, float* out_k) {
  __shared__ float acc[1024];
  const float* part = blockIdx.y ? part_k : part_q;
  float* out = blockIdx.y ? out_k : out_q;
  const int d = threadIdx.x % D, per = blockDim.x / D, j = threadIdx.x / D;
  const int64_t chunk = (n + gridDim.x - 1) / gridDim.x;
  const int64_t r0 = (int64_t)blockIdx.x * chunk, r1 = min(n, r0 + chunk);
  float s = 0.f;
  for (int64_t r = r0 + j; r < r1; r += per) s += part[r * D + d];
  acc[threadIdx.x] = s;
  __syncthreads();
  if (j == 0) {
    for (int k = 1; k < per; ++k) s += acc[k * D + d];
    out[(int64_t)blockIdx.x * D + d] = s;
  }
}

template <int D, bool F32>
hipError_t launch_bwd(const PrologueBwdArgs& a, hipStream_t stream) {
  const int threads = ((a.Hq + a.Hkv) * (D / 16) + 63) / 64 * 64;
  const size_t lds = a.dwq_part ? (size_t)(a.Hq + a.Hkv) * D * sizeof(float) : 0;
  hipLaunchKernelGGL((prologue_bwd_kernel<D, F32>), dim3((unsigned)((int64_t)a.B * a.S)), dim3(threads), lds,
                     stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prologue_bwd(const PrologueBwdArgs& a, hipStream_t stream) {
  if (a.D == 128) return a.f32 ? launch_bwd<128, true>(a, stream) : launch_bwd<128, false>(a, stream);
  return a.f32 ? launch_bwd<64, true>(a, stream) : launch_bwd<64, false>(a, stream);
}

int dw_scratch_floats(int D) { return 2 * kDwBlocks * D; }

hipError_t launch_dw_reduce(const float* part_q, const float* part_k, int64_t n, int D, float* scratch, float* dw_q,
                            float* dw_k, hipStream_t stream) {
  if (n == 0) {  // empty sums: one pass over no rows writes the zeros
    hipLaunchKernelGGL(dw_sum_kernel, dim3(1, 2), dim3(1024), 0, stream, part_q, part_k, n, D, dw_q, dw_k);
    return hipGetLastError();
  }
  float* sq = scratch;
  float* sk = scratch + (int64_t)kDwBlocks * D;
  hipLaunchKernelGGL(dw_sum_kernel, dim3(kDwBlocks, 2), dim3(1024), 0, stream, part_q, part_k, n, D, sq, sk);
  hipLaunchKernelGGL(dw_sum_kernel, dim3(1, 2), dim3(1024), 0, stream, (const float*)sq, (const float*)sk,
                     (int64_t)kDwBlocks, D, dw_q, dw_k);
  return hipGetLastError();
}

}  // namespace ha

// ====================================================================== debug position check
// HA_DEBUG only: the first position outside [0, n_pos), found with a 64-bit atomic minimum
// over the flat index (the kernels themselves clamp positions to that range).
namespace ha {
namespace {

__device__ unsigned long long g_first_bad_position;

__global__ void reset_position_check() { g_first_bad_position = ~0ull; }

__global__ __launch_bounds__(256) void position_check_kernel(const int32_t* pos, int64_t count, int32_t n_pos) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += (int64_t)gridDim.x * blockDim.x) {
    const int32_t v = pos[i];
    if (v < 0 || v >= n_pos) atomicMin(&g_first_bad_position, (unsigned long long)i);
  }
}

}  // namespace

hipError_t check_positions(const int32_t* positions, int64_t count, int32_t n_pos, hipStream_t stream,
                           int64_t* first_bad, int32_t* value) {
  *first_bad = -1;
  *value = 0;
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(reset_position_check, dim3(1), dim3(1), 0, stream);
  const int64_t blocks = std::min<int64_t>((count + 255) / 256, 1024);
  hipLaunchKernelGGL(position_check_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, positions, count, n_pos);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  unsigned long long bad = 0;
  e = hipMemcpyFromSymbolAsync(&bad, HIP_SYMBOL(g_first_bad_position), sizeof bad, 0, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess || bad == ~0ull) return e;
  *first_bad = (int64_t)bad;
  e = hipMemcpyAsync(value, positions + bad, sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  return e;
}

}  // namespace ha
