// Flash-style hybrid-mask GQA attention for gfx950 (CDNA4).
//
// out[b,i,h] = sum_j softmax_j(scale * q[b,i,h] . k[b,j,g]) v[b,j,g] over the keys j the
// row may attend to, g = h / (Hq/Hkv). Every row's keys form a prefix [0, lim(i)) (see
// ha_classify.hip), so a query block only visits key tiles [0, kend) and applies the
// per-element mask j < lim(i) only on tiles [kfull, kend) and on a ragged last tile.
// (Mask rules: HiDream-O1 atlas page, "How it works"; hidream-o1-p100a model card, "What
// this model is"; HunyuanImage 3.0 digest, "Generalized Causal Attention". GQA 32/8,
// head dim 128: model card architecture paragraph.)
//
// Work item: one (batch, KV head, query block). Its waves cover the G query heads that
// share the KV head, 32 query rows per wave, so every K/V tile staged in LDS serves all
// G heads. Per 64-key tile each wave computes
//   S^T (keys x rows)  = K Q^T   with v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q)
//   O^T (dims x rows) += V^T P^T with the same instruction    (A = V^T from LDS, B = P)
// In this orientation one lane holds one query row (lane % 32) and 16 of every 32 keys,
// so the online-softmax row max and row sum are in-lane plus one permlane32 swap, and
// the S^T accumulator registers are already the B operand of the second product: the
// accumulator of 32x32 MFMA puts key 8*(r/4) + 4*(lane/32) + r%4 in register r, and the
// staged V^T permutes each 16-key group's 4-key chunks as [0, 2, 1, 3] so the A operand
// matches that key order.
// Softmax: exp2 with scale*log2(e) folded in, fp32 running max and sum, O rescaled only
// when some row's max grew. P is rounded to bf16 for the second product (fp32 inputs
// keep P in fp32 and use v_mfma_f32_32x32x2_f32).
#include <type_traits>

#include "ha_internal.h"

namespace ha {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kHi = 1048576.0f;             // 2^20: largest tile row sum taken as is
constexpr float kLo = 8.673617379884035e-19f; // 2^-60: smallest running row sum taken as is
constexpr bf16x2 kOnes = {(__bf16)1.0f, (__bf16)1.0f};

constexpr int BK = kBlockK;

constexpr int tsub_for(int group) { return group == 1 ? 4 : (group == 2 ? 2 : 1); }

template <int D, int G, bool F32>
struct Cfg {
  static constexpr int TSUB = tsub_for(G);   // 32-row slices per head
  static constexpr int NW = G * TSUB;        // waves per work item
  static constexpr int NT = NW * 64;
  static constexpr int BQ = 32 * TSUB;       // query tokens per work item
  using T = std::conditional_t<F32, float, __bf16>;
  // bf16: K [BK][D+8], V^T [D][BK+8] (16-byte rows padded so 32 lanes reading 32 rows
  // at one column hit distinct banks). fp32: K and V [BK][D+1].
  static constexpr int KP = F32 ? D + 1 : D + 8;
  static constexpr int VP = F32 ? D + 1 : BK + 8;
  static constexpr int K_ELEMS = BK * KP;
  static constexpr int V_ELEMS = F32 ? BK * VP : D * VP;
  static constexpr int BUF = K_ELEMS + V_ELEMS;
  // bf16 staging: K as 16-byte chunks, V as (4 keys x 8 dims) blocks
  static constexpr int KCH = (BK * D / 8 + NT - 1) / NT;
  static constexpr int VTASKS = (BK / 4) * (D / 8);
  static constexpr int VT = (VTASKS + NT - 1) / NT;
};

__device__ inline float wave_pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                            __builtin_bit_cast(unsigned, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}

__device__ inline float wave_pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                            __builtin_bit_cast(unsigned, x), false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// P = exp2(S) (S in log2 units when q is prescaled, else scaled by c here) for one
// 64-key tile, rounded to bf16 in the B-operand order of the second product; returns the
// lane's sum of the rounded values (two keys per v_dot2, two chains).
template <bool PRE>
__device__ inline float exp_tile(const f32x16 (&s)[2], float c, bf16x8 (&pf)[4]) {
#pragma unroll
  for (int KS = 0; KS < 4; ++KS)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = s[KS >> 1][(KS & 1) * 8 + e];
      pf[KS][e] = static_cast<__bf16>(__builtin_amdgcn_exp2f(PRE ? x : x * c));
    }
  float t0 = 0.f, t1 = 0.f;
#pragma unroll
  for (int KS = 0; KS < 4; ++KS)
#pragma unroll
    for (int t = 0; t < 4; t += 2) {
      const bf16x2 p0 = {pf[KS][2 * t], pf[KS][2 * t + 1]};
      const bf16x2 p1 = {pf[KS][2 * t + 2], pf[KS][2 * t + 3]};
      t0 = __builtin_amdgcn_fdot2_f32_bf16(p0, kOnes, t0, false);
      t1 = __builtin_amdgcn_fdot2_f32_bf16(p1, kOnes, t1, false);
    }
  return t0 + t1;
}

// Position of key kk (0..BK-1) inside a staged V^T row: chunks of 4 keys within each
// 16-key group are stored in the order [0, 2, 1, 3].
__device__ inline int vt_pos(int kk) {
  const int c4 = (kk >> 2) & 3;
  const int nc4 = (c4 == 1) ? 2 : (c4 == 2 ? 1 : c4);
  return (kk & ~15) | (nc4 << 2) | (kk & 3);
}

template <int D, int G, bool F32>
struct Stage {
  using C = Cfg<D, G, F32>;
  bf16x8 kr[C::KCH];
  bf16x8 vr[C::VT][4];
  const __bf16* kbase;  // k and v of this (batch, KV head) at key 0 (uniform)
  const __bf16* vbase;
  int64_t tile_stride;  // elements between consecutive key tiles
  int rows_left0;       // S
  int koff[C::KCH];     // per-thread element offsets inside a tile
  int voff[C::VT];

  __device__ inline void init(const AttnArgs& a, int b, int g) {
    const int rs = a.Hkv * D;  // elements between consecutive keys
    kbase = static_cast<const __bf16*>(a.k) + ((int64_t)b * a.S * a.Hkv + g) * D;
    vbase = static_cast<const __bf16*>(a.v) + ((int64_t)b * a.S * a.Hkv + g) * D;
    tile_stride = (int64_t)BK * rs;
    rows_left0 = a.S;
    const int tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < C::KCH; ++j) {
      const int c = tid + j * C::NT;
      koff[j] = (c / (D / 8)) * rs + 8 * (c % (D / 8));
    }
#pragma unroll
    for (int j = 0; j < C::VT; ++j) {
      const int t = tid + j * C::NT;
      voff[j] = 4 * (t % (BK / 4)) * rs + 8 * (t / (BK / 4));
    }
  }

  // Global -> registers for key tile kb. Only a tile that runs past the sequence end
  // (RAGGED) checks rows; its missing rows are zero.
  template <bool RAGGED>
  __device__ inline void load(int kb) {
    const int tid = threadIdx.x;
    const __bf16* kt = kbase + kb * tile_stride;
    const __bf16* vt = vbase + kb * tile_stride;
    const int left = rows_left0 - kb * BK;  // keys of this tile inside the sequence
    const int rs = (int)(tile_stride / BK);
    const bf16x8 zero = {};
#pragma unroll
    for (int j = 0; j < C::KCH; ++j) {
      const int c = tid + j * C::NT;
      const bool ok = (C::KCH * C::NT == BK * D / 8 || c < BK * D / 8) && (!RAGGED || c / (D / 8) < left);
      kr[j] = ok ? *reinterpret_cast<const bf16x8*>(kt + koff[j]) : zero;
    }
#pragma unroll
    for (int j = 0; j < C::VT; ++j) {
      const int t = tid + j * C::NT;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool ok = (C::VT * C::NT == C::VTASKS || t < C::VTASKS) &&
                        (!RAGGED || 4 * (t % (BK / 4)) + u < left);
        vr[j][u] = ok ? *reinterpret_cast<const bf16x8*>(vt + voff[j] + u * rs) : zero;
      }
    }
  }

  __device__ inline void load_tile(int kb) {
    if ((kb + 1) * BK <= rows_left0)
      load<false>(kb);
    else
      load<true>(kb);
  }

  __device__ inline void commit(__bf16* buf) {
    const int tid = threadIdx.x;
    __bf16* ks = buf;
    __bf16* vt = buf + C::K_ELEMS;
    for (int j = 0; j < C::KCH; ++j) {
      const int c = tid + j * C::NT;
      if (C::KCH * C::NT == BK * D / 8 || c < BK * D / 8) {
        const int key = c / (D / 8), dc = c % (D / 8);
        *reinterpret_cast<bf16x8*>(ks + key * C::KP + 8 * dc) = kr[j];
      }
    }
    for (int j = 0; j < C::VT; ++j) {
      const int t = tid + j * C::NT;
      if (C::VT * C::NT == C::VTASKS || t < C::VTASKS) {
        const int kg = t % (BK / 4), dc = t / (BK / 4);
        const int pos = vt_pos(4 * kg);
        // 4 keys x 8 dims -> 8 rows of 4 consecutive keys, on 32-bit words (two bf16 each)
        const u32x4 w0 = __builtin_bit_cast(u32x4, vr[j][0]), w1 = __builtin_bit_cast(u32x4, vr[j][1]);
        const u32x4 w2 = __builtin_bit_cast(u32x4, vr[j][2]), w3 = __builtin_bit_cast(u32x4, vr[j][3]);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const u32x2 even = {(w0[m] & 0xFFFFu) | (w1[m] << 16), (w2[m] & 0xFFFFu) | (w3[m] << 16)};
          const u32x2 odd = {(w0[m] >> 16) | (w1[m] & 0xFFFF0000u), (w2[m] >> 16) | (w3[m] & 0xFFFF0000u)};
          *reinterpret_cast<u32x2*>(vt + (8 * dc + 2 * m) * C::VP + pos) = even;
          *reinterpret_cast<u32x2*>(vt + (8 * dc + 2 * m + 1) * C::VP + pos) = odd;
        }
      }
    }
  }
};

template <int D, int G, bool F32, bool PRE>
__global__ __launch_bounds__((Cfg<D, G, F32>::NT), 2) void attn_kernel(AttnArgs a) {
  using C = Cfg<D, G, F32>;
  using T = typename C::T;
  __shared__ __attribute__((aligned(16))) T lds[(F32 ? 1 : 2) * C::BUF];

  // ---- work item: XCD-aware order when the (batch, KV head) pairs split evenly over
  // the 8 XCDs (workgroups go round-robin to XCDs), so each XCD's L2 keeps the K/V of
  // its own pairs; query blocks run from the last to the first (the cheap causal text
  // blocks at the front of the sequence finish the grid).
  const int nbg = a.B * a.Hkv;
  const int item = blockIdx.x;
  int bg, slot;
  if (nbg % 8 == 0) {
    const int xcd = item % 8, s = item / 8;
    bg = xcd + 8 * (s / a.nq);
    slot = s % a.nq;
  } else {
    bg = item / a.nq;
    slot = item % a.nq;
  }
  const int qb = a.nq - 1 - slot;
  const int b = bg / a.Hkv, g = bg % a.Hkv;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hg = wave % G, tsub = wave / G;
  const int h = g * G + hg;
  const int hi = lane >> 5;
  const int S = a.S;
  const int i = qb * C::BQ + tsub * 32 + (lane & 31);
  const bool row_ok = i < S;
  const int ic = row_ok ? i : S - 1;
  const int lim = row_ok ? a.row_limit[(int64_t)b * S + i] : S;
  const int kfull = a.ranges[((int64_t)b * a.nq + qb) * 2 + 0];
  const int kend = a.ranges[((int64_t)b * a.nq + qb) * 2 + 1];
  const float c = a.scale_log2e;
  const int64_t qrow = (((int64_t)b * S + ic) * a.Hq + h) * D;

  f32x16 o[D / 32];
  for (int mt = 0; mt < D / 32; ++mt) o[mt] = f32x16{};
  float lfinal;

  if constexpr (!F32) {
    // Softmax state of this lane's row, in log2 units: reference m (not necessarily the
    // running max) and l = sum of exp2(score - m) over the row's keys seen so far. negm holds -m in the
    // units of the S accumulator (log2 units when q is prescaled, raw otherwise) and is
    // the C operand of each tile's first MFMA, so the subtraction costs nothing.
    float m = 0.f, l = 0.f;
    f32x16 negm = f32x16{};
    const __bf16* qp = static_cast<const __bf16*>(a.q);
    bf16x8 qf[D / 16];
    for (int ks = 0; ks < D / 16; ++ks)
      qf[ks] = *reinterpret_cast<const bf16x8*>(qp + qrow + 16 * ks + 8 * hi);

    Stage<D, G, F32> st;
    st.init(a, b, g);
    st.load_tile(0);
    st.commit(lds);
    __syncthreads();

    for (int kb = 0; kb < kend; ++kb) {
      const __bf16* ks_lds = lds + (kb & 1) * C::BUF;
      const __bf16* vt_lds = ks_lds + C::K_ELEMS;
      const bool more = kb + 1 < kend;
      if (more) st.load_tile(kb + 1);

      // S^T - m for the two 32-key halves, interleaved so the chains overlap
      f32x16 s[2];
      {
        const __bf16* krow = ks_lds + (lane & 31) * C::KP + 8 * hi;
        const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(krow);
        const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(krow + 32 * C::KP);
        s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[0], negm, 0, 0, 0);
        s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[0], negm, 0, 0, 0);
#pragma unroll
        for (int kk = 1; kk < D / 16; ++kk) {
          const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(krow + 16 * kk);
          const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(krow + 32 * C::KP + 16 * kk);
          s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b0, qf[kk], s[0], 0, 0, 0);
          s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b1, qf[kk], s[1], 0, 0, 0);
        }
      }

      if (kb >= kfull || (kb + 1) * BK > S) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kb * BK + 32 * kt + 8 * (r >> 2) + 4 * hi + (r & 3);
            s[kt][r] = key >= lim ? -INFINITY : s[kt][r];
          }
      }

      // Fast path: P = exp2(S - m) as is. It is taken unless some row's tile sum leaves
      // [kLo, kHi] (or is not finite), in which case those rows are re-referenced first;
      // either way numerator and denominator share the reference, so the result is the
      // softmax up to rounding.
      // A row lives in two lanes (one per 16-key half of every 32 keys) and their O^T
      // registers hold different output dims accumulated from both halves' P, so the
      // row's state (l, m, the re-reference decision) is kept whole in both lanes: the
      // tile sum is reduced over the pair first.
      bf16x8 pf[4];
      float ts = wave_pair_sum(exp_tile<PRE>(s, c, pf));
      const bool bad = !(ts <= kHi) || !(l + ts >= kLo);
      if (__builtin_amdgcn_ballot_w64(bad)) {
        float mx = s[0][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
        mx = wave_pair_max(mx);
        if (!PRE) mx *= c;
        // new reference (relative to m): the larger of the tile max and log2(l), so both
        // the old sum and the new tile end up <= 1 and at least one of them near 1
        float sh = fmaxf(mx, __builtin_amdgcn_logf(l));
        sh = (bad && sh > -INFINITY) ? sh : 0.f;
        m += sh;
        // alpha <= 1/l for l > 0 (sh >= log2 l), and l >= 2^-60 outside the first tile, so
        // it cannot overflow; with l = 0 nothing has been accumulated (O = 0) and it is 0
        const float alpha = l == 0.f ? 0.f : __builtin_amdgcn_exp2f(-sh);
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) o[mt] *= alpha;
        l *= alpha;
        const float shs = PRE ? sh : sh / c;  // in accumulator units
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          negm[r] -= shs;
          s[0][r] -= shs;
          s[1][r] -= shs;
        }
        ts = wave_pair_sum(exp_tile<PRE>(s, c, pf));
      }
      l += ts;

      // O^T += V^T P^T
#pragma unroll
      for (int KS = 0; KS < BK / 16; ++KS) {
        const __bf16* vrow = vt_lds + (lane & 31) * C::VP + 16 * KS + 8 * hi;
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) {
          const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vrow + 32 * mt * C::VP);
          o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[KS], o[mt], 0, 0, 0);
        }
      }

      if (more) st.commit(lds + ((kb + 1) & 1) * C::BUF);
      __syncthreads();
    }
    lfinal = l;
  } else {
    // fp32 inputs: plain online softmax with the running max, fp32 P.
    float m = -INFINITY, l = 0.f;
    const float cs = PRE ? 1.f : c;
    const float* qp = static_cast<const float*>(a.q);
    const float* kp = static_cast<const float*>(a.k);
    const float* vp = static_cast<const float*>(a.v);
    float qf[D / 2];
    for (int kk = 0; kk < D / 2; ++kk) qf[kk] = qp[qrow + 2 * kk + hi];

    for (int kb = 0; kb < kend; ++kb) {
      float* ks_lds = lds;
      float* v_lds = lds + C::K_ELEMS;
      __syncthreads();
      for (int e = tid; e < BK * D; e += C::NT) {
        const int key = e / D, d = e % D;
        const int gk = kb * BK + key;
        const int64_t off = (((int64_t)b * S + gk) * a.Hkv + g) * D + d;
        ks_lds[key * C::KP + d] = gk < S ? kp[off] : 0.f;
        v_lds[key * C::VP + d] = gk < S ? vp[off] : 0.f;
      }
      __syncthreads();

      f32x16 s[2];
      for (int kt = 0; kt < 2; ++kt) {
        s[kt] = f32x16{};
        const float* krow = ks_lds + (32 * kt + (lane & 31)) * C::KP + hi;
        for (int kk = 0; kk < D / 2; ++kk)
          s[kt] = __builtin_amdgcn_mfma_f32_32x32x2f32(krow[2 * kk], qf[kk], s[kt], 0, 0, 0);
      }
      if (kb >= kfull || (kb + 1) * BK > S) {
        for (int kt = 0; kt < 2; ++kt)
          for (int r = 0; r < 16; ++r) {
            const int key = kb * BK + 32 * kt + 8 * (r >> 2) + 4 * hi + (r & 3);
            if (key >= lim) s[kt][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
      for (int kt = 0; kt < 2; ++kt)
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
      mx = wave_pair_max(mx);
      const float mnew = fmaxf(m, mx);
      const float mc = (mnew == -INFINITY) ? 0.f : mnew * cs;
      const float alpha = (mnew == -INFINITY) ? 1.f : exp2f(m * cs - mc);
      for (int mt = 0; mt < D / 32; ++mt) o[mt] *= alpha;
      l *= alpha;
      m = mnew;
      for (int kt = 0; kt < 2; ++kt)
        for (int r = 0; r < 16; ++r) {
          const float p = exp2f(s[kt][r] * cs - mc);
          s[kt][r] = p;
          l += p;
        }
      // B operand of step t (two keys): register t of each lane half, i.e. key
      // 32kt + 8(t/4) + 4*half + t%4; the A operand reads V at the same keys.
      for (int kt = 0; kt < 2; ++kt)
        for (int t = 0; t < 16; ++t) {
          const int key = 32 * kt + 8 * (t >> 2) + 4 * hi + (t & 3);
          const float* vrow = v_lds + key * C::VP + (lane & 31);
          for (int mt = 0; mt < D / 32; ++mt)
            o[mt] = __builtin_amdgcn_mfma_f32_32x32x2f32(vrow[32 * mt], s[kt][t], o[mt], 0, 0, 0);
        }
    }
    lfinal = wave_pair_sum(l);  // per-lane partial sums over the two key halves
  }

  const float inv = 1.f / lfinal;
  if (row_ok) {
    const int64_t orow = (((int64_t)b * S + i) * a.Hq + h) * D;
    for (int mt = 0; mt < D / 32; ++mt)
      for (int j = 0; j < 4; ++j) {
        const int d0 = 32 * mt + 8 * j + 4 * hi;
        if constexpr (F32) {
          f32x4 w = {o[mt][4 * j] * inv, o[mt][4 * j + 1] * inv, o[mt][4 * j + 2] * inv,
                     o[mt][4 * j + 3] * inv};
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + orow + d0) = w;
        } else {
          bf16x4 w = {static_cast<__bf16>(o[mt][4 * j] * inv), static_cast<__bf16>(o[mt][4 * j + 1] * inv),
                      static_cast<__bf16>(o[mt][4 * j + 2] * inv), static_cast<__bf16>(o[mt][4 * j + 3] * inv)};
          *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(a.out) + orow + d0) = w;
        }
      }
  }
}

template <int D, int G, bool F32>
hipError_t launch(const AttnArgs& a, hipStream_t stream) {
  using C = Cfg<D, G, F32>;
  const int64_t items = (int64_t)a.B * a.Hkv * a.nq;
  if (a.q_prescaled)
    hipLaunchKernelGGL((attn_kernel<D, G, F32, true>), dim3((unsigned)items), dim3(C::NT), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_kernel<D, G, F32, false>), dim3((unsigned)items), dim3(C::NT), 0, stream, a);
  return hipGetLastError();
}

template <int D, bool F32>
hipError_t launch_g(const AttnArgs& a, hipStream_t stream) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch<D, 1, F32>(a, stream);
    case 2: return launch<D, 2, F32>(a, stream);
    case 4: return launch<D, 4, F32>(a, stream);
    default: return launch<D, 8, F32>(a, stream);
  }
}

}  // namespace

int attn_block_q(int head_dim, int group, bool f32) {
  (void)head_dim;
  (void)f32;
  return 32 * tsub_for(group);
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t stream) {
  if (a.D == 128) return a.f32 ? launch_g<128, true>(a, stream) : launch_g<128, false>(a, stream);
  return a.f32 ? launch_g<64, true>(a, stream) : launch_g<64, false>(a, stream);
}

}  // namespace ha
