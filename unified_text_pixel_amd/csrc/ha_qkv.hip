// QKV projection with the q/k prologue fused into its epilogue.
//
// Each backbone layer projects its normalised hidden states x [T][hidden] to q, k and v by
// one linear map and then normalises and rotates q and k before attention (hidream-o1-p100a
// model card, "What this model is": hidden 4096, GQA 32/8, head dim 128, q/k RMSNorm,
// mRoPE). Here y = x W^T with W [(Hq + 2 Hkv) 128][hidden] (rows: q heads, k heads, v
// heads) is computed on the matrix cores and, while each head's 128 values of a token are
// still in registers in fp32, q and k get RMSNorm (y / sqrt(mean(y^2) + eps) * w), the
// rotary embedding (pair (i, i + 64) rotated by pos[axis(i)] * theta^(-2i/128), angles
// from the caller's cos/sin table) and q its output scale; q, k and v are then written
// once in bf16 in the layouts the attention kernel reads. This saves writing the
// projection and reading it back for a separate prologue pass.
//
// Work decomposition. A workgroup computes a BM-token x BN-feature tile of y with WM x WN
// waves; a wave owns one head (128 features) and 32 MT tokens. The products run
// transposed, y^T = W x^T, on v_mfma_f32_32x32x16_bf16 with A = W rows and B = x rows, so
// a lane holds one token and 64 of its head's features (the other 64 in lane ^ 32): the
// RMSNorm sum is one cross-lane add and each rotary pair (i, i + 64) sits in one lane.
// K is walked in stages of 64: x and W rows of the stage are brought into LDS by
// global_load_lds (1 KB per instruction, 8 rows of 128 bytes), double-buffered in distinct
// arrays so the compiler never makes a read of one buffer wait for DMA into the other.
// 16-byte chunk c of LDS row r sits at c ^ (r & 7) ^ ((r >> 3) & 1): the 32 rows an
// operand read touches spread over all banks. Tiles are ordered so the workgroups that run
// together on one XCD share their x and W tiles in its L2.
#include "ha_internal.h"

namespace ha {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int HD = 128;   // head dim: one wave's features

// 16-byte chunk c of LDS row r (CPR chunks per row) is stored at c ^ swz(r). An operand read
// has 32 lanes on 32 consecutive rows at one chunk; the hardware serves 8 (128-byte rows
// of 32 banks) or 16 lanes (64 banks) at a time, and both groups land on distinct banks.
template <int CPR>
__device__ inline int swz(int r) {
  if constexpr (CPR == 8)
    return (r & 7) ^ ((r >> 3) & 1);
  else
    return ((r >> 1) & 3) ^ ((r >> 3) & 1);
}

template <int WN, int WM, int MT, int BK, int NST>
struct CfgP {
  static constexpr int NW = WN * WM;
  static constexpr int NT = 64 * NW;
  static constexpr int BN = HD * WN;         // features per workgroup
  static constexpr int BM = 32 * MT * WM;    // tokens per workgroup
  static constexpr int ROWB = BK * 2;        // bytes per LDS row
  static constexpr int CPR = BK / 8;         // chunks per row
  static constexpr int RPI = 1024 / ROWB;    // rows per 1 KB DMA instruction
  static constexpr int XBYTES = BM * ROWB;   // one stage of x
  static constexpr int WBYTES = BN * ROWB;   // one stage of W
  static constexpr int XI = XBYTES / 1024;   // DMA instructions per stage
  static constexpr int WI = WBYTES / 1024;
  static constexpr int IPW = (XI + WI) / NW; // DMA instructions per wave per stage
  static_assert(XI % NW == 0 && WI % NW == 0, "DMA instructions must split evenly over waves");
  static_assert(NST >= 3 && NST <= 5, "stage ring of 3 to 5 buffers");
  static_assert(IPW * (NST - 2) <= 63, "vmcnt range");
};

// Stage DMA of rows row0.. of a row-major bf16 matrix (ld elements per row) at column k0
// into an LDS array. Instruction ins covers LDS rows RPI ins .. RPI ins + RPI - 1; lane L
// writes row RPI ins + L / CPR at physical chunk L % CPR, which holds logical chunk
// (L % CPR) ^ swz(row). Rows past rmax read row rmax.
template <typename C, int NI>
__device__ inline void stage_dma(const __bf16* base, int64_t ld, int row0, int rmax, int k0, char* lds,
                                 int wave, int lane) {
#pragma unroll
  for (int j = 0; j < NI / C::NW; ++j) {
    // a runtime index: compile-time LDS offsets lead hipcc to an illegal constant address form
    const int ins = wave + C::NW * j;
    const int row = C::RPI * ins + lane / C::CPR;
    const int chunk = (lane % C::CPR) ^ swz<C::CPR>(row);
    const __bf16* src = base + (int64_t)min(row0 + row, rmax) * ld + k0 + 8 * chunk;
    __builtin_amdgcn_global_load_lds(src, (lds_void*)(lds + ins * 1024), 16, 0, 0);
  }
}

// Workgroup barrier without a global memory fence. __syncthreads() (and a fence on LDS
// alone, which LDS DMA also counts against) makes the compiler wait for every outstanding
// load first, the DMA of later stages included. Here the stage's own DMA is waited for
// explicitly (wait_vm) before the barrier; the wave's own LDS reads are waited for
// (lgkmcnt(0)) so that no read of a buffer is in flight once another wave refills it; the
// memory clobber keeps the compiler from moving any memory access across the barrier.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __asm__ volatile("s_barrier" ::: "memory");
}

// s_waitcnt vmcnt(N), N <= 63, lgkmcnt and expcnt not waited for (gfx9 encoding)
template <int N>
__device__ inline void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// XCD-aware, grouped tile order: blocks are dealt to the 8 XCDs in turn, so XCD x runs
// blocks x, x + 8, ...; each XCD gets a contiguous run of tile indices, walked GM token
// tiles at a time across every feature tile.
__device__ inline bool tile_of(int nM, int nN, int* m, int* n) {
  constexpr int GM = 4;
  const int total = nM * nN;
  const int per_xcd = (total + 7) / 8;
  const int u = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (u >= total) return false;
  const int group = GM * nN;
  const int g = u / group, w = u % group;
  const int first = g * GM;
  const int gm = min(nM - first, GM);
  *m = first + w % gm;
  *n = w / gm;
  return true;
}

template <int WN, int WM, int MT, int BK, int NST>
__global__ __launch_bounds__((CfgP<WN, WM, MT, BK, NST>::NT), 1) void qkv_kernel(QkvArgs a) {
  using C = CfgP<WN, WM, MT, BK, NST>;
  // the stage ring: NST buffers of x and of W, each its own array (a read of one then never
  // waits for DMA into another); unused ones shrink to 1 KB
  __shared__ __attribute__((aligned(1024))) char x0[C::XBYTES], x1[C::XBYTES], x2[C::XBYTES];
  __shared__ __attribute__((aligned(1024))) char x3[NST > 3 ? C::XBYTES : 1024];
  __shared__ __attribute__((aligned(1024))) char x4[NST > 4 ? C::XBYTES : 1024];
  __shared__ __attribute__((aligned(1024))) char w0[C::WBYTES], w1[C::WBYTES], w2[C::WBYTES];
  __shared__ __attribute__((aligned(1024))) char w3[NST > 3 ? C::WBYTES : 1024];
  __shared__ __attribute__((aligned(1024))) char w4[NST > 4 ? C::WBYTES : 1024];

  const int nM = (a.T - a.m_begin + C::BM - 1) / C::BM;
  const int n_heads = a.Hq + 2 * a.Hkv;
  const int nN = (n_heads + WN - 1) / WN;
  int mtile, ntile;
  if (!tile_of(nM, nN, &mtile, &ntile)) return;  // whole workgroup: no barrier is skipped
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % WN, wm = wave / WN;
  const int hi = lane >> 5, ln = lane & 31;
  const int m0 = a.m_begin + mtile * C::BM;     // first token of the workgroup
  const int f0 = ntile * C::BN;                 // first feature of the workgroup
  const int nfeat = n_heads * HD;
  const __bf16* xg = static_cast<const __bf16*>(a.x);
  const __bf16* wg = static_cast<const __bf16*>(a.w);
  const int K = a.K;
  const int nks = K / BK;

  f32x16 acc[4][MT];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = f32x16{};

  // operand rows of this lane: W row wn*128 + 32 nt + ln, x row wm*32 MT + 32 mt + ln
  const int wrow = wn * HD + ln;
  const int xrow = wm * 32 * MT + ln;

  auto compute = [&](const char* xb, const char* wb) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int c = 2 * kk + hi;
      bf16x8 af[4], bf[MT];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int r = wrow + 32 * nt;
        af[nt] = *reinterpret_cast<const bf16x8*>(wb + r * C::ROWB + ((c ^ swz<C::CPR>(r)) * 16));
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int r = xrow + 32 * mt;
        bf[mt] = *reinterpret_cast<const bf16x8*>(xb + r * C::ROWB + ((c ^ swz<C::CPR>(r)) * 16));
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[nt][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[nt], bf[mt], acc[nt][mt], 0, 0, 0);
    }
  };
  // Prologue DMA of a stage (in the loop, each step places its DMA between its products).
  // The scheduling barrier keeps the compiler from sinking it behind the first products.
  auto fetch = [&](int t, char* xb, char* wb) __attribute__((always_inline)) {
    stage_dma<C, C::XI>(xg, K, m0, a.T - 1, t * BK, xb, wave, lane);
    stage_dma<C, C::WI>(wg, K, f0, nfeat - 1, t * BK, wb, wave, lane);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto xbuf = [&](auto j) __attribute__((always_inline)) -> char* {
    constexpr int J = decltype(j)::value;
    if constexpr (J == 0) return x0;
    else if constexpr (J == 1) return x1;
    else if constexpr (J == 2) return x2;
    else if constexpr (J == 3) return x3;
    else return x4;
  };
  auto wbuf = [&](auto j) __attribute__((always_inline)) -> char* {
    constexpr int J = decltype(j)::value;
    if constexpr (J == 0) return w0;
    else if constexpr (J == 1) return w1;
    else if constexpr (J == 2) return w2;
    else if constexpr (J == 3) return w3;
    else return w4;
  };
  // Stage t lives in buffer t mod NST. Step t: wait until stage t has landed (the NST - 2
  // stages after it may still be in flight: vector memory completes in order), a barrier
  // (which also retires every wave's reads of buffer t - 1), the DMA of stage t + NST - 1
  // into that buffer, then stage t's products. Every step issues a DMA (past the last stage
  // it loads the last stage again into the buffer nobody reads any more): the wait count is
  // then the same at every step, and no branch around a DMA makes the compiler's own wait
  // placement fall back to waiting for all of them.
  auto step = [&](auto j, int t) __attribute__((always_inline)) {
    constexpr int J = decltype(j)::value;
    constexpr int JN = (J + NST - 1) % NST;
    wait_vm<C::IPW * (NST - 2)>();
    lds_barrier();
    {
      const int tn = min(t + NST - 1, nks - 1);
      stage_dma<C, C::XI>(xg, K, m0, a.T - 1, tn * BK, xbuf(std::integral_constant<int, JN>{}), wave, lane);
      stage_dma<C, C::WI>(wg, K, f0, nfeat - 1, tn * BK, wbuf(std::integral_constant<int, JN>{}), wave, lane);
    }
    compute(xbuf(j), wbuf(j));
    // schedule per 16-k substep: its LDS reads, then its MFMAs with the stage's DMA spread
    // between them (a burst of DMA ahead of the products stalls issue longer)
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      __builtin_amdgcn_sched_group_barrier(0x100, 4 + MT, 0);  // DS reads of the substep
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);       // MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);       // VMEM: stage DMA
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4 * MT - 4, 0);
    }
  };
  fetch(0, x0, w0);
  fetch(min(1, nks - 1), x1, w1);
  if constexpr (NST > 3) fetch(min(2, nks - 1), x2, w2);
  if constexpr (NST > 4) fetch(min(3, nks - 1), x3, w3);
  int t0 = 0;
  for (; t0 + NST <= nks; t0 += NST) {
    step(std::integral_constant<int, 0>{}, t0);
    step(std::integral_constant<int, 1>{}, t0 + 1);
    step(std::integral_constant<int, 2>{}, t0 + 2);
    if constexpr (NST > 3) step(std::integral_constant<int, 3>{}, t0 + 3);
    if constexpr (NST > 4) step(std::integral_constant<int, 4>{}, t0 + 4);
  }
  // the last nks mod NST stages
  if (t0 < nks) step(std::integral_constant<int, 0>{}, t0);
  if (t0 + 1 < nks) step(std::integral_constant<int, 1>{}, t0 + 1);
  if constexpr (NST > 3)
    if (t0 + 2 < nks) step(std::integral_constant<int, 2>{}, t0 + 2);
  if constexpr (NST > 4)
    if (t0 + 3 < nks) step(std::integral_constant<int, 3>{}, t0 + 3);
  wait_vm<0>();  // no DMA may still write this workgroup's LDS when its waves end

  // ---- epilogue: this wave's head, its lane's tokens
  const int head = ntile * WN + wn;
  if (head >= n_heads) return;
  const bool isq = head < a.Hq, isk = !isq && head < a.Hq + a.Hkv;
  const int h = isq ? head : (isk ? head - a.Hq : head - a.Hq - a.Hkv);
  const int nh = isq ? a.Hq : a.Hkv;
  __bf16* out = static_cast<__bf16*>(isq ? a.q_out : (isk ? a.k_out : a.v_out));
  const float* nw = isq ? a.wq : a.wk;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int token = m0 + wm * 32 * MT + 32 * mt + ln;
    // element (nt, r) is feature 32 nt + 8 (r / 4) + 4 hi + r % 4 of the head
    if (!isq && !isk) {
      // v: as computed
    } else {
      if (nw) {
        float ss = 0.f;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int r = 0; r < 16; ++r) ss += acc[nt][mt][r] * acc[nt][mt][r];
        ss += __shfl_xor(ss, 32);
        const float inv = 1.0f / sqrtf(ss / (float)HD + a.eps);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int f = 32 * nt + 8 * (r >> 2) + 4 * hi + (r & 3);
            acc[nt][mt][r] = acc[nt][mt][r] * inv * nw[f];
          }
      }
      if (a.rotate) {
        const int tc = min(token, a.T - 1);
        const int32_t* pos = a.positions + (int64_t)tc * a.n_axes;
        const float2* cs = reinterpret_cast<const float2*>(a.cos_sin);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int i = 32 * nt + 8 * (r >> 2) + 4 * hi + (r & 3);  // pair (i, i + 64)
            int p = pos[a.axis[i]];
            p = min(max(p, 0), a.n_pos - 1);
            const float2 t = cs[(int64_t)p * (HD / 2) + i];
            const float x1 = acc[nt][mt][r], x2 = acc[nt + 2][mt][r];
            acc[nt][mt][r] = x1 * t.x - x2 * t.y;
            acc[nt + 2][mt][r] = x2 * t.x + x1 * t.y;
          }
      }
      if (isq && a.q_scale != 1.f) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[nt][mt] *= a.q_scale;
      }
    }
    if (token < a.T) {
      __bf16* orow = out + ((int64_t)token * nh + h) * HD;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x4 v = {static_cast<__bf16>(acc[nt][mt][4 * j]), static_cast<__bf16>(acc[nt][mt][4 * j + 1]),
                            static_cast<__bf16>(acc[nt][mt][4 * j + 2]), static_cast<__bf16>(acc[nt][mt][4 * j + 3])};
          *reinterpret_cast<bf16x4*>(orow + 32 * nt + 8 * j + 4 * hi) = v;
        }
    }
  }
}

// The kernel's configurations: 2 heads x 256 tokens per workgroup (8 waves of 128 features x
// 64 tokens), and for the tail 1 head x 128 tokens (4 waves of 128 x 32, a quarter of a main
// tile, so the tail's tiles spread over about as many CUs as a round has); K in a ring of 5
// stages (three in flight behind the one computed), 32 wide for the main tile and 64 for the
// tail's (160 KB of LDS each; the wider stage gives the tail's four waves twice the products
// between two barriers).
constexpr int kWN = 2, kWM = 4, kBK = 32, kNST = 5;
constexpr int kTailWN = 1, kTailWM = 4, kTailMT = 1, kTailBK = 64;
using Main = CfgP<kWN, kWM, 2, kBK, kNST>;

template <int WN, int WM, int MT, int BK = kBK>
hipError_t launch_part(const QkvArgs& a, hipStream_t stream) {
  using C = CfgP<WN, WM, MT, BK, kNST>;
  const int nM = (a.T - a.m_begin + C::BM - 1) / C::BM;
  const int nN = (a.Hq + 2 * a.Hkv + WN - 1) / WN;
  const int total = nM * nN;
  const int grid = (total + 7) / 8 * 8;
  hipLaunchKernelGGL((qkv_kernel<WN, WM, MT, BK, kNST>), dim3((unsigned)grid), dim3(C::NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

int qkv_block_tokens() { return Main::BM; }

// One workgroup runs per CU at a time. The 256-token tiles take the tokens that fill whole
// rounds of the CUs; the tokens left over (which would run a last, mostly idle round) go to
// tiles of one head and 128 tokens, four times as many and each a quarter as long.
hipError_t launch_qkv(const QkvArgs& a, int n_cus, hipStream_t stream) {
  const int nN = (a.Hq + 2 * a.Hkv + kWN - 1) / kWN;
  const int full = a.T / Main::BM;                         // whole 256-token tiles
  const int rounds = n_cus > 0 ? full * nN / n_cus : 0;    // whole rounds they fill
  const int m_main = rounds * n_cus / nN;                  // token tiles of those rounds
  QkvArgs p = a;
  if (m_main > 0) {
    p.m_begin = 0;
    p.T = m_main * Main::BM;
    const hipError_t e = launch_part<kWN, kWM, 2>(p, stream);
    if (e != hipSuccess) return e;
  }
  if (m_main * Main::BM < a.T) {
    p = a;
    p.m_begin = m_main * Main::BM;
    return launch_part<kTailWN, kTailWM, kTailMT, kTailBK>(p, stream);
  }
  return hipSuccess;
}

}  // namespace ha
