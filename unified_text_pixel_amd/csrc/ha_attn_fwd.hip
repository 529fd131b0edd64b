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
// Work item: one (batch, KV head, query block). Its eight waves (two per SIMD) cover the G
// query heads that share the KV head, 32 query rows per wave, 256 / G rows per block, so
// every K/V tile staged in LDS serves all of them. (With fewer work items than CUs and
// G = 4, each 32-row slice of a block is a workgroup of its own, G waves, so that the
// items spread over twice as many CUs; the rows compute exactly as before.) Per 64-key tile each wave computes
//   S^T (keys x rows)  = K Q^T   with v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q)
//   O^T (dims x rows) += V^T P^T with the same instruction    (A = V^T from LDS, B = P)
// In this orientation one lane holds one query row (lane % 32) and 16 of every 32 keys
// (the accumulator of a 32x32 MFMA puts key 8*(r/4) + 4*(lane/32) + r%4 in register r),
// so the row reductions are in-lane plus one permlane32 swap, and the S^T registers,
// rounded to bf16, are already the B operand of the second product.
//
// bf16 pipeline (one barrier per key tile):
//  - K and V tiles go from global memory straight into LDS (global_load_lds_dwordx4, no
//    registers); K runs two tiles ahead and V one, in two buffers each (four distinct
//    LDS arrays).
//  - Step t computes S_{t+1}, O += V_{t-1} P_{t-1} and P_t = exp2(S_t): the exponentials
//    interleave with both MFMA chains.
//  - V stays row-major in LDS; ds_read_b64_tr_b16 gathers the transposed A operand.
//  - Both tiles are XOR-swizzled on 16-byte chunks so the reads are bank-conflict free.
// Softmax: q arrives prescaled by scale*log2(e) (or the scale is applied here) and the
// main pass keeps the reference at 0, P = exp2(S) taken as is; a work item in which some
// row's tile sum leaves [2^-60, 2^64] is redone on a careful pass that re-references
// (exactly; see below).
// fp32 inputs use a plain variant (fp32 P, v_mfma_f32_32x32x2_f32, running max).
#include <array>
#include <type_traits>

#include "ha_internal.h"

namespace ha {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr float kHi = 18446744073709551616.0f;  // 2^64: largest tile row sum taken as is
constexpr float kLo = 8.673617379884035e-19f; // 2^-60: smallest running row sum taken as is
constexpr bf16x2 kOnes = {(__bf16)1.0f, (__bf16)1.0f};

constexpr int BK = kBlockK;

// 32-row slices per query head in one work item: bf16 uses eight waves (two per SIMD, so
// every K/V tile staged in LDS serves 8 x 32 query rows), fp32 four
constexpr int tsub_for(int group) { return 8 / group; }
constexpr int tsub_f32(int group) { return group == 1 ? 4 : (group == 2 ? 2 : 1); }

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

// Work item of this workgroup: XCD-aware order when the (batch, KV head) pairs split
// evenly over the 8 XCDs (workgroups go round-robin to XCDs), so each XCD's L2 keeps the
// K/V of its own pairs; query blocks run from the last to the first (the cheap causal
// text blocks at the front of the sequence finish the grid). Only the last nq_run blocks
// of each pair are work items (all of them unless a caller reuses a step-invariant prefix).
struct Item {
  int b, g, qb;
};
__device__ inline Item work_item(const AttnArgs& a, int item) {
  const int nbg = a.B * a.Hkv;
  int bg, slot;
  if (nbg % 8 == 0) {
    const int xcd = item % 8, s = item / 8;
    bg = xcd + 8 * (s / a.nq_run);
    slot = s % a.nq_run;
  } else {
    bg = item / a.nq_run;
    slot = item % a.nq_run;
  }
  return {bg / a.Hkv, bg % a.Hkv, a.nq - 1 - slot};
}

// ====================================================================== bf16
//
// LDS tiles: BK keys x D bf16, row-major (a row is one key), 16-byte chunks XOR-swizzled
// within the row: physical chunk = logical chunk ^ swizzle(row).
//   K: swizzle = row mod (chunks per row). A K-operand read has 32 lanes on 32
//      consecutive rows at one chunk, which then spread over all banks.
//   V: swizzle = {0, 6, 10, 12}[row mod 4]. A transposing read covers 8 rows x 4
//      chunks; 16 lanes read 4 rows x 2 chunks and 32 lanes 4 rows x 4 chunks, which
//      these values place in distinct banks for 32 or 64 banks of 4 bytes.
template <int D>
struct Tile {
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int BYTES = BK * D * 2;      // one tile
  static constexpr int NI = BYTES / 1024;       // 1 KB DMA instructions per tile
  static constexpr int RPI = 1024 / (2 * D);    // rows per DMA instruction
  __device__ static inline int kswz(int row) { return row & (CPR - 1); }
  __device__ static inline int vswz(int row) { return (0xCA60 >> (4 * (row & 3))) & (CPR - 1); }
};

// WS: one workgroup per 32-row slice of a query block (G waves), so that a problem with
// fewer work items than CUs spreads over more of them; otherwise one workgroup covers the
// whole block (G * TSUB waves).
template <int D, int G, bool WS = false>
struct CfgB {
  static constexpr int TSUB = tsub_for(G);    // 32-row slices per query block
  static constexpr int WSUB = WS ? 1 : TSUB;  // slices per workgroup
  static constexpr int NW = G * WSUB;
  static constexpr int NT = NW * 64;
  static constexpr int BQ = 32 * TSUB;
  static constexpr int IPW = Tile<D>::NI / NW;  // DMA instructions per wave per tile and tensor
  static_assert(Tile<D>::NI % NW == 0, "DMA instructions must split evenly over waves");
};

// DMA of key tiles (BK rows of K or V for one batch item and KV head) into swizzled LDS
// buffers. DMA instruction ins covers tile bytes [1024 ins, +1024): lane L writes bytes
// +16 L, i.e. tile row RPI*ins + L/CPR at physical chunk L%CPR, which holds logical chunk
// (L%CPR) ^ swizzle(row). Since RPI is a multiple of 4 and L/CPR < RPI, that logical
// chunk is, for V, a per-lane constant and, for K, a per-lane constant XOR a per-
// instruction constant; the global address is a uniform base plus a per-lane offset.
// Rows past the sequence end (only in the last tile) read its last row instead: masked
// keys get P = 0 and that row is finite.
template <int D, int G, bool WS>
struct Dma {
  using TL = Tile<D>;
  const char* kbase;  // key 0 of this batch item and KV head (uniform)
  const char* vbase;
  int64_t row_bytes;  // bytes between consecutive keys
  int S, wave, lrow;  // lrow = lane / CPR
  unsigned koff, kx16, voff, lane16;

  __device__ inline void init(const void* k, const void* v, int b, int g, int S_, int Hkv, int wave_,
                              int lane) {
    row_bytes = (int64_t)Hkv * D * 2;
    kbase = static_cast<const char*>(k) + ((int64_t)b * S_ * Hkv + g) * D * 2;
    vbase = static_cast<const char*>(v) + ((int64_t)b * S_ * Hkv + g) * D * 2;
    S = S_;
    wave = wave_;
    lrow = lane / TL::CPR;
    const int pc = lane % TL::CPR;
    koff = (unsigned)(lrow * row_bytes);
    kx16 = 16u * (unsigned)(pc ^ lrow);
    voff = (unsigned)(lrow * row_bytes) + 16u * (unsigned)(pc ^ TL::vswz(lrow));
    lane16 = 16u * (unsigned)pc;
  }

  // CLAMP: the tile may run past the sequence end (per-lane row clamp)
  template <bool ISV, bool CLAMP>
  __device__ inline void tile(int key0, char* buf) const {
#pragma unroll
    for (int j = 0; j < CfgB<D, G, WS>::IPW; ++j) {
      const int ins = wave * CfgB<D, G, WS>::IPW + j;
      const char* src;
      if constexpr (!CLAMP) {
        const char* g = (ISV ? vbase : kbase) + (key0 + TL::RPI * ins) * row_bytes;
        const unsigned u = 16u * (unsigned)((TL::RPI * ins) & (TL::CPR - 1));
        src = g + (ISV ? voff : koff + (kx16 ^ u));
      } else {
        const int rr = TL::RPI * ins + lrow;
        const int c = (int)(lane16 / 16u) ^ (ISV ? TL::vswz(rr) : TL::kswz(rr));
        src = (ISV ? vbase : kbase) + min(key0 + rr, S - 1) * row_bytes + 16 * c;
      }
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(buf + ins * 1024), 16, 0, 0);
    }
  }
};

// LM, the list mode: 0, the work item walks tiles [0, kend) of its query block, tile t at
// position t.
//   LM & 1  (a layout with Gen Images) it walks the query block's tile list instead (inside
//           FULL tiles first, then the rest), and masked tiles also hide keys whose
//           visibility ends at or before the row;
//   LM & 2  work items come from a table: a query block may be split into parts, each
//           walking a share of the positions and writing unnormalised partial results that
//           combine_kernel merges.
template <int D, int G, bool PRE, bool LSE, int LM, bool WS = false>
__global__ __launch_bounds__((CfgB<D, G, WS>::NT), 2) void attn_bf16(AttnArgs a) {
  constexpr bool KVIS = (LM & 1) != 0, ITEMS = (LM & 2) != 0, LIST = KVIS;
  static_assert(!WS || LM == 0, "slice workgroups walk plain tile ranges");
  using C = CfgB<D, G, WS>;
  using TL = Tile<D>;
  // K and V double buffers as four distinct arrays: a read of one buffer then never waits
  // for DMA still landing in another (the compiler tracks LDS DMA per array)
  __shared__ __attribute__((aligned(1024))) char k0[TL::BYTES];
  __shared__ __attribute__((aligned(1024))) char k1[TL::BYTES];
  __shared__ __attribute__((aligned(1024))) char v0[TL::BYTES];
  __shared__ __attribute__((aligned(1024))) char v1[TL::BYTES];
  __shared__ int redo;  // some row left the range on the main pass: redo the work item

  int b, g, qb, part = 0, nparts = 1, slot = -1;
  if constexpr (ITEMS) {
    const int32_t* itm = a.items + (int64_t)blockIdx.x * 4;
    const int bg = itm[0];
    if (bg < 0) return;  // padding entry: the whole workgroup leaves before any barrier
    b = bg / a.Hkv;
    g = bg % a.Hkv;
    qb = itm[1];
    part = itm[2] & 0xffff;
    nparts = itm[2] >> 16;
    slot = itm[3];
  }
  int wslice = 0;  // WS: this workgroup's 32-row slice of the block
  if constexpr (!ITEMS) {
    int item = blockIdx.x;
    if constexpr (WS) {
      // the slices of a work item go to one XCD (workgroups go round-robin to the 8 XCDs),
      // one after the other in dispatch order
      if ((a.B * a.Hkv) % 8 == 0) {
        wslice = (item / 8) % C::TSUB;
        item = (item / (8 * C::TSUB)) * 8 + item % 8;
      } else {
        wslice = item % C::TSUB;
        item /= C::TSUB;
      }
    }
    const Item it = work_item(a, item);
    b = it.b;
    g = it.g;
    qb = it.qb;
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hg = wave % G, tsub = WS ? wslice : wave / G;
  const int h = g * G + hg;
  const int hi = lane >> 5;
  const int S = a.S;
  // query blocks end at S (the first block of the sequence is the ragged one)
  const int i = S - (a.nq - qb) * C::BQ + tsub * 32 + (lane & 31);
  const bool row_ok = i >= 0;
  const int ic = row_ok ? i : 0;
  const int lim = row_ok ? a.row_limit[(int64_t)b * S + i] : S;
  // positions [0, kfull) of the walk are unmasked, [kfull, kend) masked; position t is
  // key tile tile_at(t)
  const int32_t* cnt = LIST ? a.tile_count : a.ranges;
  int kfull = cnt[((int64_t)b * a.nq + qb) * 2 + 0];
  int kend = cnt[((int64_t)b * a.nq + qb) * 2 + 1];
  const int32_t* tlist = LIST ? a.tiles + ((int64_t)b * a.nq + qb) * a.nk : nullptr;
  int t0 = 0;  // tile at position 0 (without a list)
  if constexpr (ITEMS) {
    if (nparts > 1) {  // part p of the walk: positions [p n / P, (p + 1) n / P)
      const int p0 = (int)((int64_t)part * kend / nparts), p1 = (int)((int64_t)(part + 1) * kend / nparts);
      if constexpr (LIST)
        tlist += p0;
      else
        t0 = p0;
      kfull = min(max(kfull - p0, 0), p1 - p0);
      kend = p1 - p0;
    }
    if (kend <= 0) {  // an empty part: it saw no key (the merge skips it)
      if (hi == 0) a.part_l[((int64_t)slot * C::BQ + tsub * 32 + (lane & 31)) * G + hg] = 0.f;
      return;
    }
  }
  // The tile list is written before the launch and only read here: read through the
  // constant address space, it takes scalar loads (a plain load is a vector load, whose wait
  // would also wait for the tile DMA just issued).
  auto tile_at = [&](int t) __attribute__((always_inline)) {
    if constexpr (LIST)
      return ((const __attribute__((address_space(4))) int32_t*)tlist)[t];
    else if constexpr (ITEMS)
      return t0 + t;
    else
      return t;
  };
  const float c = a.scale_log2e;
  Dma<D, G, WS> dma;
  dma.init(a.k, a.v, b, g, S, a.Hkv, wave, lane);

  // K-operand reads: row 32kt + (lane & 31), logical chunk 2kk + hi
  const int krow = lane & 31;
  const int kx = hi ^ TL::kswz(krow);  // chunk 2kk + hi sits at (2kk) ^ kx
  // V-operand transposing reads: lane t of 16-lane group G16 points at key
  // 16KS + 8rr + 4(G16 >> 1) + t/4 and dims 32mt + 16(G16 & 1) + 4(t & 3) (8 bytes)
  const int g16 = lane >> 4, t16 = lane & 15;
  const int vrow = 4 * (g16 >> 1) + (t16 >> 2);  // + 16KS + 8rr, which keep row mod 4
  const int vclow = 2 * (g16 & 1) + ((t16 & 3) >> 1);
  const int vx = vclow ^ TL::vswz(vrow);  // chunk 4mt + vclow sits at (4mt) ^ vx
  const int vhalf = 8 * (t16 & 1);

  // Softmax state of this lane's row, in log2 units: reference m and l = sum of
  // exp2(score - m) over the row's keys seen so far. A row lives in two lanes (one per
  // 16-key half of every 32 keys) whose O^T registers hold different output dims
  // accumulated from both halves' P, so the row's state is kept whole in both lanes (tile
  // sums are reduced over the pair). The main pass keeps m = 0 throughout: P = exp2(S)
  // needs no subtraction and no running max. A lane only records whether a tile sum of
  // its row left [kLo, kHi] (or was not finite); if any did, the work item is redone on
  // a careful pass that re-references (below).
  float l = 0.f;
  f32x16 o[D / 32];
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) o[mt] = f32x16{};

  const __bf16* qp = static_cast<const __bf16*>(a.q) + (((int64_t)b * S + ic) * a.Hq + h) * D;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qp + 16 * ks + 8 * hi);
  // A training forward (row lse) of q without the scale takes q' = bf16(scale log2(e) q),
  // rounded as the prologue rounds it: the backward rebuilds P from those same q' values and
  // this lse, so both must score with the same q' (with the scale applied in fp32 here
  // instead, a large component common to every key would shift each row's scores by the
  // rounding of q' between the two passes, and P's rows would no longer sum to 1)
  constexpr bool PS = PRE || LSE;  // scores in log2 units: q prescaled, given or made here
  if constexpr (!PRE && LSE) {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[ks][e] = static_cast<__bf16>(static_cast<float>(qf[ks][e]) * c);
  }

  // S^T + c0 for the 64 keys of a K buffer, the two 32-key halves interleaved (c0 is the
  // C operand of the first MFMA: zero, or -m on the careful pass)
  auto qk = [&](const char* kbuf, const f32x16& c0) {
    std::array<f32x16, 2> s;
    // the lane's row offset and chunk swizzle, opaque: each k-step's address is rebuilt
    // with one XOR instead of D/16 offsets held live across the loop
    int kro = krow * (2 * D), kx16 = kx * 16;
    __asm__ volatile("" : "+v"(kro), "+v"(kx16));
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const int off = kro + ((32 * kk) ^ kx16);
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(kbuf + off);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(kbuf + off + 32 * 2 * D);
      s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[kk], kk == 0 ? c0 : s[0], 0, 0, 0);
      s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[kk], kk == 0 ? c0 : s[1], 0, 0, 0);
    }
    return s;
  };

  // Masks the tile at position t of S (keys >= lim, and with Gen Images keys whose
  // visibility ends at or before row i) where the tile is partial or runs past the end.
  // With work items from a table or Gen Images it returns whether the lane's row sees a key
  // of the tile (a part of a split block can hold tiles that some of its rows cannot see
  // yet, and a tile list can start with tiles hidden from some rows).
  constexpr bool TRACK = ITEMS || KVIS;
  auto mask = [&](f32x16 (&sc)[2], int t) {
    const int tile = tile_at(t);
    if (t < kfull && (tile + 1) * BK <= S) return true;
    bool any = false;
    if constexpr (KVIS) {
      // the lane's keys come in runs of 4: key_vis rows are padded, so every run is in bounds
      const int* kv = a.key_vis + (int64_t)b * a.kv_stride + tile * BK + 4 * hi;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const i32x4 vis = *reinterpret_cast<const i32x4*>(kv + 32 * kt + 8 * q4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * q4 + e;
            const int key = tile * BK + 32 * kt + 8 * q4 + 4 * hi + e;
            const bool hide = key >= lim || i >= vis[e];
            if constexpr (TRACK) any = any || !hide;
            sc[kt][r] = hide ? -INFINITY : sc[kt][r];
          }
        }
      if constexpr (TRACK) {  // the row's other 32 keys sit in the partner lane (lane ^ 32)
        const auto r = __builtin_amdgcn_permlane32_swap((unsigned)any, (unsigned)any, false, false);
        any = (r[0] | r[1]) != 0;
      }
    } else {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = tile * BK + 32 * kt + 8 * (r >> 2) + 4 * hi + (r & 3);
          sc[kt][r] = key >= lim ? -INFINITY : sc[kt][r];
        }
      any = lim > tile * BK;  // the tile's keys are contiguous from tile * BK
    }
    return any;
  };

  // O^T += V^T P^T for one tile; the A operand of K step KS, dims 32mt.. comes from two
  // transposing reads (keys +0..3 and +8..11 of the lane's half)
  auto pv = [&](const char* vb, const bf16x8 (&pf)[4]) {
    // per dims block mt the lane's offset, opaque (the buffer + one register + a constant
    // per K step), rebuilt per call rather than held live across the loop
    int vo[D / 32];
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt) {
      vo[mt] = vrow * (2 * D) + (((4 * mt) ^ vx) * 16) + vhalf;
      __asm__ volatile("" : "+v"(vo[mt]));
    }
    auto rdv = [&](int j) __attribute__((always_inline)) {
      const int KS = j / (D / 32), mt = j % (D / 32);
      const char* p0 = vb + vo[mt] + 16 * KS * (2 * D);
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p0);
      const bf16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0 + 8 * 2 * D));
      return __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    // the A operand of product j + 1 is read while product j runs
    constexpr int NJ = (BK / 16) * (D / 32);
    bf16x8 vf[2];
    vf[0] = rdv(0);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (j + 1 < NJ) vf[(j + 1) & 1] = rdv(j + 1);
      const int KS = j / (D / 32), mt = j % (D / 32);
      o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[j & 1], pf[KS], o[mt], 0, 0, 0);
    }
  };

  // One main-pass step for tile t: land K_{t+1} and V_{t-1}, start the DMA of K_{t+2}
  // and V_t, then S_{t+1} = K_{t+1} Q^T, O += V_{t-1} P_{t-1} and P_t = exp2(S_t). Tile
  // j sits in buffer j mod 2 (PAR = t mod 2, known at compile time). FAST steps (tiles
  // t-1 .. t+2 present, tiles t .. t+2 full and inside the sequence) have no branch at
  // all, so the two MFMA chains and the exponentials interleave freely.
  bool off_range = false;
  bool seen = false;  // (table work items, Gen Images) the row has seen a key of its walk
  auto step = [&](auto fast_tag, auto par_tag, int t, f32x16 (&sc)[2], f32x16 (&sn)[2],
                  bf16x8 (&pfp)[4], bf16x8 (&pf)[4]) {
    constexpr bool FAST = decltype(fast_tag)::value;
    constexpr int PAR = decltype(par_tag)::value;
    char* const kw = PAR ? k1 : k0;        // K_t, free now: receives K_{t+2}
    const char* const kr = PAR ? k0 : k1;  // K_{t+1}
    char* const vw = PAR ? v1 : v0;        // receives V_t
    const char* const vr = PAR ? v0 : v1;  // V_{t-1}
    // publish whether a row of this wave has left the range; read, past the barrier, whether
    // any wave has (the FAST loop stops at the end of the trip that sees it)
    if (PAR == 1 && __builtin_amdgcn_ballot_w64(off_range)) redo = 1;
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (FAST || t + 2 < kend) dma.template tile<false, !FAST>(tile_at(t + 2) * BK, kw);
    dma.template tile<true, !FAST>(tile_at(t) * BK, vw);
    if (FAST || t + 1 < kend) {
      const auto s1 = qk(kr, f32x16{});
      sn[0] = s1[0];
      sn[1] = s1[1];
    }
    if (FAST || t >= 1) pv(vr, pfp);
    bool vis = true;
    if (!FAST) vis = mask(sc, t);
    const float ts = wave_pair_sum(exp_tile<PS>(sc, c, pf));
    if constexpr (TRACK) {
      // a row that has seen no key of its part yet has nothing to be out of range
      seen = seen || vis;
      off_range = off_range || !(ts <= kHi) || (seen && !(l + ts >= kLo));
    } else {
      off_range = off_range || !(ts <= kHi) || !(l + ts >= kLo);
    }
    l += ts;
    // read past the barrier, at the end of the step: no wave publishes again before the
    // next odd step's barrier, which every wave reaches only after this read
    return PAR == 1 && __builtin_amdgcn_readfirstlane(redo) != 0;
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;

  if (tid == 0) redo = 0;
  // prologue: K0 and K1 in flight, S_0 (the barrier also publishes redo = 0)
  dma.template tile<false, true>(tile_at(0) * BK, k0);
  if (kend > 1) dma.template tile<false, true>(tile_at(1) * BK, k1);
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  // P_t sits in register set t mod 2 (pa, pb)
  f32x16 sa[2], sb[2] = {f32x16{}, f32x16{}};
  bf16x8 pa[4], pb[4];
  {
    const auto s0 = qk(k0, f32x16{});
    sa[0] = s0[0];
    sa[1] = s0[1];
  }

  // tiles [1, fast_end) take the FAST step: tile t is full and inside the sequence, and
  // so is tile t + 2 (DMA without clamping). Both loops take two steps per trip (odd t,
  // then even), the S registers alternating roles; sb holds S_t when a trip starts. (A
  // tile list puts the tiles that are full and inside the sequence first.)
  const int fast_end = LIST ? max(1, min(kfull, kend) - 2) : max(1, min(min(kfull, kend - 2), S / BK - t0 - 2));
  // Once a row of the work item has left the range the main pass stops at the end of the
  // FAST trip that sees it (the careful pass below starts over), so a work item that needs
  // the careful pass wastes little of its main pass.
  step(std::false_type{}, P0{}, 0, sa, sb, pb, pa);  // S_1 -> sb, P_0 -> pa
  int t = 1;
  bool left = false;
  for (; t + 1 < fast_end && !left; t += 2) {
    left = step(std::true_type{}, P1{}, t, sb, sa, pa, pb);  // S_{t+1} -> sa, P_t -> pb
    step(std::true_type{}, P0{}, t + 1, sa, sb, pb, pa);     // S_{t+2} -> sb, P_{t+1} -> pa
  }
  for (; !left && t + 1 < kend; t += 2) {
    step(std::false_type{}, P1{}, t, sb, sa, pa, pb);
    step(std::false_type{}, P0{}, t + 1, sa, sb, pb, pa);
  }
  if (!left && t < kend) step(std::false_type{}, P1{}, t, sb, sa, pa, pb);
  // last tile's P V (a main pass left early computes a P V the careful pass discards)
  if (__builtin_amdgcn_ballot_w64(off_range)) redo = 1;
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if ((kend - 1) & 1)
    pv(v1, pb);
  else
    pv(v0, pa);

  // Careful pass, only when some row of the work item left the range: every wave starts
  // over and re-references rows whose tile sum leaves [kLo, kHi] to the larger of the tile
  // max and log2(l), so both the old sum and the new tile end up <= 1 with one of them near
  // 1. Numerator and denominator share the reference either way, so the result is the
  // softmax up to rounding. negm holds -m in the units of the S accumulator (log2 units
  // when q is prescaled, raw otherwise) and is the C operand of each tile's first MFMA.
  // Tile u sits in buffer u mod 2 (compile-time parity) and tile u + 1's DMA runs while
  // tile u is computed; past the last tile the DMA reloads the last tile into the free
  // buffer, which nothing reads (a DMA behind a branch would make the compiler wait for
  // every DMA in flight before the next LDS read).
  float mref = 0.f;  // the row's reference m (0 unless the careful pass moved it)
  if (redo) {
    f32x16 negm = f32x16{};
    l = 0.f;
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt) o[mt] = f32x16{};
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // every wave is done with the buffers
    dma.template tile<false, true>(tile_at(0) * BK, k0);
    dma.template tile<true, true>(tile_at(0) * BK, v0);
    auto cstep = [&](auto par_tag, int u) __attribute__((always_inline)) {
      constexpr int PAR = decltype(par_tag)::value;
      const char* const kb = PAR ? k1 : k0;
      const char* const vb = PAR ? v1 : v0;
      char* const kn = PAR ? k0 : k1;
      char* const vn = PAR ? v0 : v1;
      __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();  // tile u landed; every wave is done with tile u - 1's buffers
      const int un = min(u + 1, kend - 1);
      dma.template tile<false, true>(tile_at(un) * BK, kn);
      dma.template tile<true, true>(tile_at(un) * BK, vn);
      const auto s0 = qk(kb, negm);
      f32x16 sc[2] = {s0[0], s0[1]};
      mask(sc, u);
      float ts = wave_pair_sum(exp_tile<PS>(sc, c, pa));
      const bool bad = !(ts <= kHi) || !(l + ts >= kLo);
      if (__builtin_amdgcn_ballot_w64(bad)) {
        float mx = sc[0][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[0][r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[1][r]);
        mx = wave_pair_max(mx);
        if (!PS) mx *= c;
        float sh = fmaxf(mx, __builtin_amdgcn_logf(l));
        sh = (bad && sh > -INFINITY) ? sh : 0.f;
        mref += sh;
        // alpha <= 1/l for l > 0 (sh >= log2 l), and l >= kLo outside the first tile, so
        // it cannot overflow; with l = 0 nothing has been accumulated (O = 0) and it is 0
        const float alpha = l == 0.f ? 0.f : __builtin_amdgcn_exp2f(-sh);
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) o[mt] *= alpha;
        l *= alpha;
        const float shs = PS ? sh : sh / c;  // in accumulator units
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          negm[r] -= shs;
          sc[0][r] -= shs;
          sc[1][r] -= shs;
        }
        ts = wave_pair_sum(exp_tile<PS>(sc, c, pa));
      }
      l += ts;
      pv(vb, pa);
    };
    int u = 0;
    for (; u + 1 < kend; u += 2) {
      cstep(P0{}, u);
      cstep(P1{}, u + 1);
    }
    if (u < kend) cstep(P0{}, u);
  }

  // a part of a split query block: its unnormalised output, row sum and row reference
  if constexpr (ITEMS) {
    if (slot >= 0) {
      const int64_t r = (int64_t)slot * C::BQ + tsub * 32 + (lane & 31);
      float* po = a.part_o + (r * G + hg) * D;
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<f32x4*>(po + 32 * mt + 8 * j + 4 * hi) =
              f32x4{o[mt][4 * j], o[mt][4 * j + 1], o[mt][4 * j + 2], o[mt][4 * j + 3]};
      if (hi == 0) {
        a.part_l[r * G + hg] = l;
        a.part_m[r * G + hg] = mref;
      }
      return;
    }
  }
  // row log-sum-exp of the natural-unit scores for a training backward: with the scores in
  // log2 units, log2 sum_j 2^s_j = m + log2(l)
  if constexpr (LSE) {
    if (i >= a.row_begin && hi == 0)
      a.lse[((int64_t)b * a.Hq + h) * S + i] = (mref + __builtin_amdgcn_logf(l)) * 0.693147180559945309f;
  }
  // The output rows go through LDS (the K/V buffers, free once every wave is past its last
  // tile), so that the global stores write whole 2D-byte rows: stored from the MFMA layout,
  // one row per lane, every store instruction would touch a cache line per lane. Wave w
  // stages its 32 rows in half of buffer w / 2, 16-byte chunks XOR-swizzled by the row.
  {
    constexpr int CPR = TL::CPR;
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    char* stg = (wave >> 1) == 0 ? k0 : ((wave >> 1) == 1 ? k1 : ((wave >> 1) == 2 ? v0 : v1));
    stg += (wave & 1) * 32 * (2 * D);
    const float inv = 1.f / l;
    const int rw = lane & 31;
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x4 w = {static_cast<__bf16>(o[mt][4 * j] * inv), static_cast<__bf16>(o[mt][4 * j + 1] * inv),
                          static_cast<__bf16>(o[mt][4 * j + 2] * inv), static_cast<__bf16>(o[mt][4 * j + 3] * inv)};
        const int chunk = (4 * mt + j) ^ (rw & (CPR - 1));  // dims 32mt + 8j .. +7
        *reinterpret_cast<bf16x4*>(stg + rw * (2 * D) + chunk * 16 + 8 * hi) = w;
      }
    // lane L stores chunk L mod CPR of row 64/CPR k + L / CPR
    constexpr int RPI = 64 / CPR;
    const int lr = lane / CPR, lc = lane % CPR;
    const int row0 = S - (a.nq - qb) * C::BQ + tsub * 32;
#pragma unroll
    for (int k = 0; k < 32 / RPI; ++k) {
      const int r = RPI * k + lr;
      const bf16x8 v8 = *reinterpret_cast<const bf16x8*>(stg + r * (2 * D) + ((lc ^ (r & (CPR - 1))) * 16));
      if (row0 + r >= a.row_begin)  // also excludes rows before the sequence (row_begin >= 0)
        *reinterpret_cast<bf16x8*>(static_cast<__bf16*>(a.out) + (((int64_t)b * S + row0 + r) * a.Hq + h) * D +
                                   8 * lc) = v8;
    }
  }
}

// ====================================================================== fp32
// Plain online softmax with the running max and fp32 P, K and V staged through
// registers into padded LDS rows, v_mfma_f32_32x32x2_f32 for both products.
template <int D, int G>
struct CfgF {
  static constexpr int TSUB = tsub_f32(G);
  static constexpr int NW = G * TSUB;
  static constexpr int NT = NW * 64;
  static constexpr int BQ = 32 * TSUB;
  static constexpr int P = D + 1;  // padded row (floats)
};

template <int D, int G, bool PRE>
__global__ __launch_bounds__((CfgF<D, G>::NT), 1) void attn_f32(AttnArgs a) {
  using C = CfgF<D, G>;
  __shared__ float ks_lds[BK * C::P];
  __shared__ float v_lds[BK * C::P];

  const Item it = work_item(a, blockIdx.x);
  const int b = it.b, g = it.g, qb = it.qb;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hg = wave % G, tsub = wave / G;
  const int h = g * G + hg;
  const int hi = lane >> 5;
  const int S = a.S;
  // query blocks end at S (the first block of the sequence is the ragged one)
  const int i = S - (a.nq - qb) * C::BQ + tsub * 32 + (lane & 31);
  const bool row_ok = i >= 0;
  const int ic = row_ok ? i : 0;
  const int lim = row_ok ? a.row_limit[(int64_t)b * S + i] : S;
  // with Gen Images the block walks its tile list (positions < kfull unmasked)
  const bool hole = a.tiles != nullptr;
  const int32_t* cnt = hole ? a.tile_count : a.ranges;
  const int kfull = cnt[((int64_t)b * a.nq + qb) * 2 + 0];
  const int kend = cnt[((int64_t)b * a.nq + qb) * 2 + 1];
  const int32_t* tlist = hole ? a.tiles + ((int64_t)b * a.nq + qb) * a.nk : nullptr;
  const float cs = PRE ? 1.f : a.scale_log2e;

  f32x16 o[D / 32];
  for (int mt = 0; mt < D / 32; ++mt) o[mt] = f32x16{};
  float m = -INFINITY, l = 0.f;
  const float* qp = static_cast<const float*>(a.q) + (((int64_t)b * S + ic) * a.Hq + h) * D;
  const float* kp = static_cast<const float*>(a.k);
  const float* vp = static_cast<const float*>(a.v);
  float qf[D / 2];
  for (int kk = 0; kk < D / 2; ++kk) qf[kk] = qp[2 * kk + hi];

  for (int pos = 0; pos < kend; ++pos) {
    const int kb = hole ? tlist[pos] : pos;
    __syncthreads();
    for (int e = tid; e < BK * D; e += C::NT) {
      const int key = e / D, d = e % D;
      const int gk = kb * BK + key;
      const int64_t off = (((int64_t)b * S + gk) * a.Hkv + g) * D + d;
      ks_lds[key * C::P + d] = gk < S ? kp[off] : 0.f;
      v_lds[key * C::P + d] = gk < S ? vp[off] : 0.f;
    }
    __syncthreads();

    f32x16 s[2];
    for (int kt = 0; kt < 2; ++kt) {
      s[kt] = f32x16{};
      const float* krow = ks_lds + (32 * kt + (lane & 31)) * C::P + hi;
      for (int kk = 0; kk < D / 2; ++kk)
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x2f32(krow[2 * kk], qf[kk], s[kt], 0, 0, 0);
    }
    if (pos >= kfull || (kb + 1) * BK > S) {
      for (int kt = 0; kt < 2; ++kt)
        for (int r = 0; r < 16; ++r) {
          const int key = kb * BK + 32 * kt + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (key >= lim || (hole && i >= a.key_vis[(int64_t)b * a.kv_stride + key])) s[kt][r] = -INFINITY;
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
        const float* vrow = v_lds + key * C::P + (lane & 31);
        for (int mt = 0; mt < D / 32; ++mt)
          o[mt] = __builtin_amdgcn_mfma_f32_32x32x2f32(vrow[32 * mt], s[kt][t], o[mt], 0, 0, 0);
      }
  }

  const float inv = 1.f / wave_pair_sum(l);  // per-lane partial sums over the two key halves
  if (i >= a.row_begin) {  // also excludes rows before the sequence (row_begin >= 0)
    float* orow = static_cast<float*>(a.out) + (((int64_t)b * S + i) * a.Hq + h) * D;
    for (int mt = 0; mt < D / 32; ++mt)
      for (int j = 0; j < 4; ++j) {
        const f32x4 w = {o[mt][4 * j] * inv, o[mt][4 * j + 1] * inv, o[mt][4 * j + 2] * inv,
                         o[mt][4 * j + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + 32 * mt + 8 * j + 4 * hi) = w;
      }
  }
}

// ====================================================================== launch
template <int D, int G, int LM>
void launch_bf16(const AttnArgs& a, dim3 grid, hipStream_t stream) {
  const dim3 block(CfgB<D, G>::NT);
  if constexpr (LM == 0 && G == 4) {
    if (a.slices > 1) {
      using C = CfgB<D, G, true>;
      const dim3 wgrid(grid.x * C::TSUB), wblock(C::NT);
      if (a.lse) {
        if (a.q_prescaled)
          hipLaunchKernelGGL((attn_bf16<D, G, true, true, LM, true>), wgrid, wblock, 0, stream, a);
        else
          hipLaunchKernelGGL((attn_bf16<D, G, false, true, LM, true>), wgrid, wblock, 0, stream, a);
      } else if (a.q_prescaled) {
        hipLaunchKernelGGL((attn_bf16<D, G, true, false, LM, true>), wgrid, wblock, 0, stream, a);
      } else {
        hipLaunchKernelGGL((attn_bf16<D, G, false, false, LM, true>), wgrid, wblock, 0, stream, a);
      }
      return;
    }
  }
  if (a.lse) {
    if (a.q_prescaled)
      hipLaunchKernelGGL((attn_bf16<D, G, true, true, LM>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((attn_bf16<D, G, false, true, LM>), grid, block, 0, stream, a);
  } else if (a.q_prescaled) {
    hipLaunchKernelGGL((attn_bf16<D, G, true, false, LM>), grid, block, 0, stream, a);
  } else {
    hipLaunchKernelGGL((attn_bf16<D, G, false, false, LM>), grid, block, 0, stream, a);
  }
}

template <int D, int G>
hipError_t launch(const AttnArgs& a, hipStream_t stream) {
  const int64_t items = a.items ? a.n_items : (int64_t)a.B * a.Hkv * a.nq_run;
  const dim3 grid((unsigned)items);
  if (a.f32) {
    const dim3 block(CfgF<D, G>::NT);
    if (a.q_prescaled)
      hipLaunchKernelGGL((attn_f32<D, G, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((attn_f32<D, G, false>), grid, block, 0, stream, a);
  } else {
    // list mode: key visibility with Gen Images, an item table for split query blocks
    const int lm = (a.key_vis ? 1 : 0) | (a.items ? 2 : 0);
    switch (lm) {
      case 1: launch_bf16<D, G, 1>(a, grid, stream); break;
      case 2: launch_bf16<D, G, 2>(a, grid, stream); break;
      case 3: launch_bf16<D, G, 3>(a, grid, stream); break;
      default: launch_bf16<D, G, 0>(a, grid, stream); break;
    }
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_g(const AttnArgs& a, hipStream_t stream) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch<D, 1>(a, stream);
    case 2: return launch<D, 2>(a, stream);
    case 4: return launch<D, 4>(a, stream);
    default: return launch<D, 8>(a, stream);
  }
}

}  // namespace

int attn_slices(int head_dim, int group, bool f32) {
  (void)head_dim;
  return (!f32 && group == 4) ? tsub_for(group) : 1;
}

int attn_block_q(int head_dim, int group, bool f32) {
  (void)head_dim;
  return 32 * (f32 ? tsub_f32(group) : tsub_for(group));
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t stream) {
  return a.D == 128 ? launch_g<128>(a, stream) : launch_g<64>(a, stream);
}

// ====================================================================== merge of split parts
// A query block split into P parts has, per row and head, P unnormalised outputs O_p, row
// sums l_p and references m_p (log2 units: the part's exponentials are exp2(s - m_p)).
// With M = max m_p over the parts that saw a key (l_p > 0) and w_p = exp2(m_p - M):
//   out = sum_p w_p O_p / sum_p w_p l_p,   lse = ln 2 (M + log2 sum_p w_p l_p).
// Threads: one per (row, head, 8 output dims); split blocks in blockIdx.y.
namespace {
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int32_t* sp = a.splits + (int64_t)blockIdx.y * 4;
  const int bg = sp[0], qb = sp[1], s0 = sp[2], np = sp[3];
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;  // (row, head, chunk of 8 dims)
  constexpr int CH = D / 8;
  if (idx >= a.BQ * a.G * CH) return;
  const int ch = idx % CH, hg = (idx / CH) % a.G, r = idx / (CH * a.G);
  const int i = a.S - (a.nq - qb) * a.BQ + r;
  if (i < 0) return;
  float M = -INFINITY;
  for (int p = 0; p < np; ++p) {
    const int64_t e = ((int64_t)(s0 + p) * a.BQ + r) * a.G + hg;
    if (a.part_l[e] > 0.f) M = fmaxf(M, a.part_m[e]);
  }
  float L = 0.f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int p = 0; p < np; ++p) {
    const int64_t e = ((int64_t)(s0 + p) * a.BQ + r) * a.G + hg;
    const float lp = a.part_l[e];
    if (!(lp > 0.f)) continue;
    const float w = __builtin_amdgcn_exp2f(a.part_m[e] - M);
    L += w * lp;
    const f32x4* po = reinterpret_cast<const f32x4*>(a.part_o + e * D + 8 * ch);
    const f32x4 u = po[0], v = po[1];
    for (int k = 0; k < 4; ++k) {
      acc[k] += w * u[k];
      acc[4 + k] += w * v[k];
    }
  }
  const float inv = 1.f / L;
  const int h = g * a.G + hg;
  __bf16* orow = static_cast<__bf16*>(a.out) + (((int64_t)b * a.S + i) * a.Hq + h) * D + 8 * ch;
  bf16x8 o;
  for (int k = 0; k < 8; ++k) o[k] = static_cast<__bf16>(acc[k] * inv);
  *reinterpret_cast<bf16x8*>(orow) = o;
  if (a.lse && ch == 0) a.lse[((int64_t)b * a.Hq + h) * a.S + i] = (M + __builtin_amdgcn_logf(L)) * 0.693147180559945309f;
}
}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  if (a.n_splits == 0) return hipSuccess;
  const int threads = a.BQ * a.G * (a.D / 8);
  const dim3 grid((unsigned)((threads + 255) / 256), (unsigned)a.n_splits);
  if (a.D == 128)
    hipLaunchKernelGGL((combine_kernel<128>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((combine_kernel<64>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ha
