// Backward of the hybrid-mask GQA attention for gfx950 (CDNA4).
//
// For a loss with output gradient dO (row i attends the key prefix [0, lim(i)); query head
// h shares KV head g; Z_ij = scale q_i . k_j; P = softmax of Z over the row's keys):
//   dV_j  = sum over the heads h of g and rows i of  P_ij dO_i        dP_ij = dO_i . v_j
//   dZ_ij = P_ij (dP_ij - delta_i),   delta_i = dO_i . O_i
//   dQ_i  = scale sum_j dZ_ij k_j,    dK_j = scale sum over h and i of dZ_ij q_i
// This is the derivative of the forward in ha_attn_fwd.hip: the pages train the models
// end to end (HiDream-O1 atlas page, "How it works"; HunyuanImage 3.0 digest, training
// stages) but print no backward. P is rebuilt from the forward's row log-sum-exp,
// P_ij = exp(Z_ij - lse_i); q comes in as q' = scale log2(e) q (the prologue's prescaled
// output), so q' . k is Z in log2 units and P = exp2(q' . k - log2(e) lse).
//
// bwd_dkdv: one workgroup per (batch, KV head, block of 256/HPS keys), HPS heads per step
//   (HPS = G, or 2 of G = 4 on large shapes). Wave w serves head slot w%HPS and keys
//   32*(w/HPS) .. +32 of the block. Per step of 32 query rows and HPS heads (the G/HPS head
//   groups of a row block in turn) the q' and dO rows are copied into LDS (global_load_lds,
//   double-buffered). In the orientation S = Q' K^T (v_mfma_f32_32x32x16_bf16, A = q'
//   rows, B = K^T, both from LDS) a lane holds one key and 16 of the 32 rows, so P and dZ
//   rounded to bf16 are already the A operand of dV += P^T dO and dK += dZ^T Q', whose B
//   operands are the dO and q' rows gathered in the same row order by ds_read_b64_tr_b16.
//   A row's lse, delta and limit come from the lane that loaded them (ds_bpermute). At the
//   end the HPS head slots' partial sums meet in LDS.
// bwd_dq: the forward's shape: one workgroup per (batch, KV head, query block), one lane
//   per query row. Per 64-key tile S^T = K Q'^T and dP^T = V dO^T (A from LDS, B = the
//   row's q' and dO held in registers); dZ^T, rounded to bf16, is the B operand of
//   dQ^T += K^T dZ^T (A = K^T gathered from LDS by ds_read_b64_tr_b16).
// bwd_delta: delta = rowsum(dO * O) in fp32.
//
// LDS tiles are row-major with 16-byte chunks XOR-swizzled by swz(row) (below); a step
// tile of q' or dO keeps the G heads of one row side by side.
#include <algorithm>
#include <type_traits>

#include "ha_internal.h"

namespace ha {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int BK = kBlockK;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.693147180559945309417f;

__device__ inline f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ inline float bpermute(int src_lane, float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * src_lane, __builtin_bit_cast(int, x)));
}

// Chunk swizzle of tile row r: physical chunk = logical chunk ^ swz(r). The tiles are read
// two ways. A row read has 16 lanes on 16 consecutive rows at one logical chunk, so swz must
// be a bijection on r mod 16. A transposing read (ds_read_b64_tr_b16) has 32 lanes on 4
// consecutive rows (4a .. 4a + 3) x 4 logical chunks (4m .. 4m + 3). With d = 128 (16
// chunks, 256 bytes: every bank once) swz(r) = (r mod 16) ^ 4 (r mod 4) sends row 4a + i to
// chunks 4(m ^ a ^ i) + (c ^ i), 16 distinct, where r mod 16 alone gives 4 chunks
// (a 4-way bank conflict). d = 64 keeps r mod 8.
template <int CPR>
__device__ inline int swz(int row) {
  return (row & (CPR - 1)) ^ (CPR == 16 ? (row & 3) << 2 : 0);
}

// Copies rows [row0, row0 + rows) of a row-major global tensor (row stride gstride bytes,
// rows clamped to [0, rmax]) into LDS, ROWB bytes per row made of segments of D elements
// (one per head), each swizzled by the row within the tile. 1 KB per DMA instruction:
// lane L writes bytes 16L of it, i.e. row RPI*ins + L*16/ROWB of the tile, segment
// (L*16 % ROWB) / 2D, physical chunk L % CPR, which holds logical chunk (L % CPR) ^
// swz(row). Instruction ins is issued by wave ins mod 8; the lane's part of the address is
// computed once.
template <int D, int ROWB, int NINS>
struct RowDma {
  static constexpr int CPR = D / 8;
  static constexpr int RPI = 1024 / ROWB;  // rows per instruction
  int rho, segb, pc;                        // the lane's row in an instruction, segment bytes, chunk

  __device__ inline void init(int lane) {
    rho = (16 * lane) / ROWB;
    segb = ((16 * lane) % ROWB) / (2 * D) * (2 * D);
    pc = ((16 * lane) % (2 * D)) / 16;
  }

  __device__ __attribute__((always_inline)) inline void issue(const char* gbase, int64_t gstride, int row0,
                                                                int rmax, char* lds, int wave) const {
    const char* tbase = gbase + (int64_t)row0 * gstride;
#pragma unroll
    for (int j = 0; j < (NINS + 7) / 8; ++j) {
      const int ins = wave + 8 * j;  // run-time: keeps the LDS address out of constant folding
      if (NINS % 8 != 0 && ins >= NINS) continue;
      const int row = ins * RPI + rho;
      const int r = min(max(row0 + row, 0), rmax);
      // a uniform tile base plus a 32-bit lane offset (r >= row0 for row0 <= rmax, and the
      // offset spans a tile), which the DMA takes as an SGPR base and one VGPR
      const unsigned off = (unsigned)((r - row0) * (int)gstride) + segb + ((pc ^ swz<CPR>(row)) * 16);
      __builtin_amdgcn_global_load_lds(tbase + off, (lds_void*)(lds + ins * 1024), 16, 0, 0);
    }
  }
};

// s_waitcnt vmcnt(0) through the builtin, so the compiler's own wait tracking knows that
// every vector memory operation has completed (gfx9 encoding: expcnt 7, lgkmcnt 15)
__device__ __attribute__((always_inline)) inline void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// (batch * KV heads) pair and block slot of workgroup x: XCD-aware when the pairs split
// evenly over the 8 XCDs (workgroups go round-robin to XCDs), so each XCD's L2 holds the
// tensors of its own pairs.
__device__ inline void pair_slot(int x, int nbg, int nblocks, int* bg, int* slot) {
  if (nbg % 8 == 0) {
    const int xcd = x % 8, s = x / 8;
    *bg = xcd + 8 * (s / nblocks);
    *slot = s % nblocks;
  } else {
    *bg = x / nblocks;
    *slot = x % nblocks;
  }
}

// ====================================================================== delta
template <int D>
__global__ __launch_bounds__(256) void bwd_delta(const __bf16* out, const __bf16* dout, float* delta, int B, int S,
                                                 int Hq) {
  constexpr int LPR = D / 8;  // lanes per (token, head) row, 8 elements each
  const int64_t n = (int64_t)B * S * Hq;
  const int64_t r = ((int64_t)blockIdx.x * 256 + threadIdx.x) / LPR;
  const int c = threadIdx.x % LPR;
  float s = 0.f;
  if (r < n) {
    const bf16x8 o = *reinterpret_cast<const bf16x8*>(out + r * D + 8 * c);
    const bf16x8 g = *reinterpret_cast<const bf16x8*>(dout + r * D + 8 * c);
#pragma unroll
    for (int e = 0; e < 8; ++e) s += static_cast<float>(o[e]) * static_cast<float>(g[e]);
  }
#pragma unroll
  for (int o = LPR / 2; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (r < n && c == 0) {
    const int h = (int)(r % Hq);
    const int64_t bi = r / Hq;
    delta[((bi / S) * Hq + h) * S + bi % S] = s;
  }
}

// ====================================================================== dK, dV
template <int D, int G, int HPS>
struct CfgKV {
  static constexpr int NS = 8 / HPS;              // 32-key slices per work item
  static constexpr int KB = 32 * NS;              // keys per work item
  static constexpr int CPR = D / 8;               // 16-byte chunks per head row
  static constexpr int QROWB = HPS * D * 2;       // one step row: HPS heads' q' (or dO)
  static constexpr int QBYTES = 32 * QROWB;       // one step tile (32 rows)
  static constexpr int KVBYTES = KB * D * 2;      // the item's K (or V) rows
  static constexpr int SUB = 8 / G;               // 32-row steps per query block
  static constexpr int NHP = G / HPS;             // steps (head groups) per 32 rows
};

// HOLE: a layout with Gen Images. Each lane's key carries its visibility (the rows below
// it see the key), and the block's smallest and largest visibility bound the steps: rows
// at or after the largest see none of the block's keys, rows at or after the smallest need
// the per-pair mask.
template <int D, int G, bool HOLE, int HPS>
__global__ __launch_bounds__(512, 2) void bwd_dkdv(BwdArgs a) {
  using C = CfgKV<D, G, HPS>;
  __shared__ __attribute__((aligned(1024))) char kt[C::KVBYTES];
  __shared__ __attribute__((aligned(1024))) char vt[C::KVBYTES];
  __shared__ __attribute__((aligned(1024))) char q0[C::QBYTES];
  __shared__ __attribute__((aligned(1024))) char q1[C::QBYTES];
  __shared__ __attribute__((aligned(1024))) char o0[C::QBYTES];
  __shared__ __attribute__((aligned(1024))) char o1[C::QBYTES];

  const int S = a.S, nq = a.nq;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hs = wave % HPS, ksl = wave / HPS;  // head slot of a step, 32-key slice
  const int hi = lane >> 5, ln = lane & 31;
  const int nkb = (a.k_end - a.k_begin + C::KB - 1) / C::KB;
  int bg, slot;
  pair_slot(blockIdx.x, a.B * a.Hkv, nkb * a.n_parts, &bg, &slot);
  const int kbk = slot / a.n_parts, part = slot % a.n_parts;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int k0 = a.k_begin + kbk * C::KB;
  const int key = k0 + 32 * ksl + ln;  // this lane's key (lanes l and l + 32 share it)
  const int BQ = 32 * C::SUB;          // rows of a forward query block
  const int qrow0 = S - nq * BQ;       // first row of query block 0 (end-aligned blocks)

  // Gen Images: the lane key's visibility, and its range over the block's keys inside the
  // sequence (every wave reduces all of them, so the bounds are uniform without LDS;
  // loaded before any DMA is issued, so using them waits for nothing else)
  int kv = S, kvmin = S, kvmax = S;
  if constexpr (HOLE) {
    const int32_t* kvb = a.key_vis + (int64_t)b * a.kv_stride;
    kv = kvb[key];  // key < key_vis_stride(S): blocks of KB keys tile it
    int lo = S, hi_ = 0;
#pragma unroll
    for (int j = 0; j < C::KB / 64; ++j) {
      const int kj = k0 + 64 * j + lane;
      const int v = kvb[kj];
      if (kj < S) {
        lo = min(lo, v);
        hi_ = max(hi_, v);
      }
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      lo = min(lo, __shfl_xor(lo, m));
      hi_ = max(hi_, __shfl_xor(hi_, m));
    }
    kvmin = __builtin_amdgcn_readfirstlane(lo);
    kvmax = __builtin_amdgcn_readfirstlane(hi_);
  }

  // the item's K and V rows
  const int64_t kvstride = (int64_t)a.Hkv * D * 2;
  const char* kbase = static_cast<const char*>(a.k) + ((int64_t)b * S * a.Hkv + g) * D * 2;
  const char* vbase = static_cast<const char*>(a.v) + ((int64_t)b * S * a.Hkv + g) * D * 2;
  {
    RowDma<D, 2 * D, C::KVBYTES / 1024> kvd;
    kvd.init(lane);
    kvd.issue(kbase, kvstride, k0, S - 1, kt, wave);
    kvd.issue(vbase, kvstride, k0, S - 1, vt, wave);
  }

  // step s = 32 rows starting at qrow0 + 32 s; active when its query block attends a key
  // >= k0 (then it attends k0: rows see prefixes) and some row is >= 0
  // this workgroup's part of the 32-row steps: [s_lo, s_hi)
  const int nsteps_all = nq * C::SUB;
  const int s_lo = (int)((int64_t)part * nsteps_all / a.n_parts);
  const int nsteps = (int)((int64_t)(part + 1) * nsteps_all / a.n_parts);
  auto next_step = [&](int s) __attribute__((always_inline)) {
    for (++s; s < nsteps; ++s) {
      if (qrow0 + 32 * s + 31 < 0) continue;
      if (HOLE && qrow0 + 32 * s >= kvmax) return -1;  // this and later rows see no key here
      const int qb = s / C::SUB;
      if (a.ranges[((int64_t)b * nq + qb) * 2 + 1] * BK > k0) return s;
      s = (qb + 1) * C::SUB - 1;
    }
    return -1;
  };

  const int64_t qstride = (int64_t)a.Hq * D * 2;
  const char* qbase = static_cast<const char*>(a.q) + ((int64_t)b * S * a.Hq + g * G) * D * 2;
  const char* obase = static_cast<const char*>(a.dout) + ((int64_t)b * S * a.Hq + g * G) * D * 2;
  const int32_t* lim_b = a.row_limit + (int64_t)b * S;
  // step s into a tile pair; the lane's row (ln) values into registers: log2(e) lse,
  // delta and the row's key limit (0 for rows before the sequence, which see no key)
  RowDma<D, C::QROWB, C::QBYTES / 1024> qd_dma;
  qd_dma.init(lane);
  // raw loads only: using a loaded value before the step's DMA has landed would make the
  // compiler wait for that DMA (vector memory operations complete in order)
  // substep u = (32-row step s, head group hp): the rows of heads g G + hp HPS .. + HPS
  auto fetch = [&](int u, char* qd, char* od, float& lr, float& dr, int& mr) __attribute__((always_inline)) {
    const int s = u / C::NHP, hp = u % C::NHP;
    const int r0 = qrow0 + 32 * s;
    const int ic = max(r0 + ln, 0);
    const int64_t hrow = ((int64_t)b * a.Hq + g * G + hp * HPS + hs) * S;
    lr = a.lse[hrow + ic];
    dr = a.delta[hrow + ic];
    mr = lim_b[ic];
    qd_dma.issue(qbase + hp * HPS * D * 2, qstride, r0, S - 1, qd, wave);
    qd_dma.issue(obase + hp * HPS * D * 2, qstride, r0, S - 1, od, wave);
  };
  auto next_sub = [&](int u) __attribute__((always_inline)) {
    if (u % C::NHP + 1 < C::NHP) return u + 1;
    const int s2 = next_step(u / C::NHP);
    return s2 < 0 ? -1 : s2 * C::NHP;
  };
  // a step needs the per-pair mask unless every row of it is inside the sequence and
  // attends every key of the block (keys [0, 64 kfull) of its query block, and < S)
  auto masked_step = [&](int s) __attribute__((always_inline)) {
    const int qb = s / C::SUB;
    const int kfull = a.ranges[((int64_t)b * nq + qb) * 2 + 0];
    return !(qrow0 + 32 * s >= 0 && k0 + C::KB <= kfull * BK && k0 + C::KB <= S) ||
           (HOLE && qrow0 + 32 * s + 31 >= kvmin);
  };

  // A/B operand reads of rows (q' or dO row ln, or K/V row 32 ksl + ln): chunk 2kk + hi of
  // the row sits at (2kk) ^ kx, kx = hi ^ swz(ln). Transposing reads: lane t of
  // 16-lane group G16 points at row 16KS + 8rr + 4(G16 >> 1) + t/4 and dims 32mt + 16(G16 & 1)
  // + 4(t & 3).

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) dk[mt] = dv[mt] = f32x16{};

  // The lane's row constants enter the first MFMA of S and of dP as an extra A column
  // (rows x 16, only k = 0, 1 used: -log2(e) lse and -delta split into bf16 hi + lo, exact
  // to 2^-16 relative) against a B column of ones, so S' = Q' K^T - log2(e) lse and
  // dP' = dO V^T - delta arrive per (row, key) without moving per-row values across lanes.
  bf16x8 ones = {};
  if (hi == 0) ones[0] = ones[1] = static_cast<__bf16>(1.0f);
  auto split_col = [&](float x) __attribute__((always_inline)) {
    bf16x8 c = {};
    const __bf16 h = static_cast<__bf16>(-x);
    if (hi == 0) {
      c[0] = h;
      c[1] = static_cast<__bf16>(-x - static_cast<float>(h));
    }
    return c;
  };

  auto compute = [&](const char* qc, const char* oc, float lr, float dr, int mr, int s, bool masked)
                     __attribute__((always_inline)) {
    // LDS addresses: a tile row's 16-byte chunk c sits at chunk c ^ swz(row), and the row
    // offset occupies the bits above the chunk, so the operand of k-step kk is at the
    // lane's k-step-0 offset XOR 32 kk. The per-lane offsets are rebuilt each step from an
    // opaque copy of the lane id (kept live across the loop they would not fit).
    int lo = lane;
    __asm__ volatile("" : "+v"(lo));
    const int lnx = lo & 31, hix = lo >> 5;
    const int kxx = hix ^ swz<C::CPR>(lnx);
    // S' and dP': rows x keys, lane = key, register r = row 8(r/4) + 4hi + r%4
    f32x16 sacc = mfma(split_col(lr * kLog2e), ones, f32x16{});
    f32x16 pacc = mfma(split_col(dr), ones, f32x16{});
    if (qrow0 + 32 * s + ln < 0) mr = 0;  // rows before the sequence see no key
    int xq = (lnx * HPS + hs) * (2 * D) + kxx * 16;   // q' and dO rows
    int xk = (32 * ksl + lnx) * (2 * D) + kxx * 16;  // K and V rows
    __asm__ volatile("" : "+v"(xq), "+v"(xk));
    auto rd = [&](const char* buf, int x, int kk) __attribute__((always_inline)) {
      return *reinterpret_cast<const bf16x8*>(buf + (x ^ (32 * kk)));
    };
    // operands of k-step kk + 1 are read while the two MFMAs of k-step kk run
    bf16x8 fq[2], fk[2], fo[2], fv[2];
    fq[0] = rd(qc, xq, 0);
    fk[0] = rd(kt, xk, 0);
    fo[0] = rd(oc, xq, 0);
    fv[0] = rd(vt, xk, 0);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const int cur = kk & 1, nxt = cur ^ 1;
      if (kk + 1 < D / 16) {
        fq[nxt] = rd(qc, xq, kk + 1);
        fk[nxt] = rd(kt, xk, kk + 1);
        fo[nxt] = rd(oc, xq, kk + 1);
        fv[nxt] = rd(vt, xk, kk + 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // the four DS reads of kk + 1
      }
      sacc = mfma(fq[cur], fk[cur], sacc);
      pacc = mfma(fo[cur], fv[cur], pacc);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);    // then the two MFMAs of kk
    }
    // P = exp2(S') on allowed (row, key) pairs, dZ = P dP'; both to bf16 with rows
    // 16KS .. 16KS + 15 in register order (the A-operand k order). Only steps that need
    // the mask fetch each row's key limit from the lane that loaded it.
    // (the mask is applied to all 16 elements in one branch: a branch per element split the
    // step into small blocks the scheduler could not interleave)
    bf16x8 pa[2], za[2];
    f32x16 pe;
#pragma unroll
    for (int r = 0; r < 16; ++r) pe[r] = __builtin_amdgcn_exp2f(sacc[r]);
    if (masked) {
      // the source lanes from an opaque copy of 4 hi, so that the compiler does not keep 16
      // loop-invariant lane addresses live across the loop
      int h4 = 4 * hi;
      __asm__ volatile("" : "+v"(h4));
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int src = 8 * (r >> 2) + h4 + (r & 3);
        const int lim = __builtin_bit_cast(int, bpermute(src, __builtin_bit_cast(float, mr)));
        pe[r] = (key < lim && (!HOLE || qrow0 + 32 * s + src < kv)) ? pe[r] : 0.f;
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      pa[r >> 3][r & 7] = static_cast<__bf16>(pe[r]);
      za[r >> 3][r & 7] = static_cast<__bf16>(pe[r] * pacc[r]);
    }
    // dV += P^T dO, dK += dZ^T Q' (B: dO / q' rows of this head gathered per dims 32mt..).
    // Transposing reads: lane t of 16-lane group G16 reads rows 16KS + 8rr + 4(G16 >> 1) + t/4
    // at chunk (4mt + vcl) ^ swz(row); rows 16KS + r share swz(r), and 4mt + vcl = 4mt ^ vcl,
    // so the address is the lane's (KS = 0, mt = 0) offset XOR 64 mt, plus KS * 16 G rows.
    const int g16x = lo >> 4, t16x = lo & 15;
    const int vrx = 4 * (g16x >> 1) + (t16x >> 2);
    const int vclx = 2 * (g16x & 1) + ((t16x & 3) >> 1);
    const int vhx = 8 * (t16x & 1);
    int tl = (vrx * HPS + hs) * (2 * D) + ((vclx ^ swz<C::CPR>(vrx)) * 16) + vhx;
    int tu = ((vrx + 8) * HPS + hs) * (2 * D) + ((vclx ^ swz<C::CPR>(vrx + 8)) * 16) + vhx;
    __asm__ volatile("" : "+v"(tl), "+v"(tu));
    // the four transposing reads of (KS, mt) + 1 are issued while the two MFMAs of (KS, mt) run
    auto trd = [&](int j, bf16x8& dvo, bf16x8& dko) __attribute__((always_inline)) {
      const int KS = j / (D / 32), mt = j % (D / 32);
      const int ks = KS * 16 * HPS * (2 * D);
      const bf16x4 dol = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(oc + ks + (tl ^ (64 * mt))));
      const bf16x4 dou = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(oc + ks + (tu ^ (64 * mt))));
      const bf16x4 qvl = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(qc + ks + (tl ^ (64 * mt))));
      const bf16x4 qvu = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(qc + ks + (tu ^ (64 * mt))));
      dvo = __builtin_shufflevector(dol, dou, 0, 1, 2, 3, 4, 5, 6, 7);
      dko = __builtin_shufflevector(qvl, qvu, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    constexpr int NJ = 2 * (D / 32);
    bf16x8 bdv[2], bdk[2];
    trd(0, bdv[0], bdk[0]);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int cur = j & 1, nxt = cur ^ 1;
      if (j + 1 < NJ) {
        trd(j + 1, bdv[nxt], bdk[nxt]);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // the four reads of j + 1
      }
      const int KS = j / (D / 32), mt = j % (D / 32);
      dv[mt] = mfma(pa[KS], bdv[cur], dv[mt]);
      dk[mt] = mfma(za[KS], bdk[cur], dk[mt]);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);    // then the two MFMAs of j
    }
  };

  // two steps per trip, tile pair (q0, o0) then (q1, o1); every step first lands its own
  // tiles (wait + barrier, which also retires every wave's reads of the pair it refills)
  float la = 0.f, da = 0.f, lb = 0.f, db = 0.f;
  int ma = 0, mb = 0;
  const int s_first = next_step(s_lo - 1);
  int u = s_first < 0 ? -1 : s_first * C::NHP;
  if (u >= 0) fetch(u, q0, o0, la, da, ma);
  while (u >= 0) {
    // the step's mask flag is read before the wait, so using it waits for nothing issued later
    const int u1 = next_sub(u);
    const bool m0 = masked_step(u / C::NHP);
    wait_vm();
    __syncthreads();
    if (u1 >= 0) fetch(u1, q1, o1, lb, db, mb);
    compute(q0, o0, la, da, ma, u / C::NHP, m0);
    if (u1 < 0) break;
    const int u2 = next_sub(u1);
    const bool m1 = masked_step(u1 / C::NHP);
    wait_vm();
    __syncthreads();
    if (u2 >= 0) fetch(u2, q0, o0, la, da, ma);
    compute(q1, o1, lb, db, mb, u1 / C::NHP, m1);
    u = u2;
  }
  wait_vm();  // K/V DMA of an item with no step

  // dK for the rotated k: scale * sum dZ q = ln(2) * sum dZ q' (q' = scale log2(e) q)
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) dk[mt] *= kLn2;

  // sum the HPS head slots' partials (waves ksl*HPS .. +HPS) through LDS, 8 registers per
  // lane per round; wave hs == 0 of each slice stores. Element (r, lane) of dv[mt] / dk[mt] is key
  // k0 + 32 ksl + 8(r/4) + 4hi + r%4, dim 32 mt + ln.
  float* red = reinterpret_cast<float*>(C::QBYTES >= 16384 ? q0 : kt);
  __bf16* dvo = static_cast<__bf16*>(a.dv) + ((int64_t)b * S * a.Hkv + g) * D;
  float* dko = a.dk + ((int64_t)b * S * a.Hkv + g) * D;
  // a part of the steps writes fp32 partial sums to its slot, keys relative to k_begin
  const int nkeys = a.k_end - a.k_begin;
  float* pdv = a.part_dv ? a.part_dv + (((int64_t)part * a.B + b) * nkeys * a.Hkv + g) * D : nullptr;
  float* pdk = a.part_dk ? a.part_dk + (((int64_t)part * a.B + b) * nkeys * a.Hkv + g) * D : nullptr;
  auto emit = [&](int which, int mt, int half, const float (&x)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int r = 8 * half + e;
      const int kj = k0 + 32 * ksl + 8 * (r >> 2) + 4 * hi + (r & 3);
      if (kj >= a.k_end) continue;
      if (pdv) {
        const int64_t at = (int64_t)(kj - a.k_begin) * a.Hkv * D + 32 * mt + ln;
        (which == 0 ? pdv : pdk)[at] = x[e];
        continue;
      }
      const int64_t at = (int64_t)kj * a.Hkv * D + 32 * mt + ln;
      if (which == 0)
        dvo[at] = static_cast<__bf16>(x[e]);
      else
        dko[at] = x[e];
    }
  };
#pragma unroll
  for (int which = 0; which < 2; ++which)
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const f32x16& acc = which == 0 ? dv[mt] : dk[mt];
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = acc[8 * half + e];
        if constexpr (HPS > 1) {
          __syncthreads();  // the previous round's (or the last step's) reads are done
          f32x4* w = reinterpret_cast<f32x4*>(red + (wave * 64 + lane) * 8);
          w[0] = f32x4{x[0], x[1], x[2], x[3]};
          w[1] = f32x4{x[4], x[5], x[6], x[7]};
          __syncthreads();
          if (hs == 0) {
#pragma unroll
            for (int o = 1; o < HPS; ++o) {
              const f32x4* rd = reinterpret_cast<const f32x4*>(red + ((wave + o) * 64 + lane) * 8);
              const f32x4 u = rd[0], v = rd[1];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                x[e] += u[e];
                x[4 + e] += v[e];
              }
            }
            emit(which, mt, half, x);
          }
        } else {
          emit(which, mt, half, x);
        }
      }
}

// ====================================================================== dQ
template <int D, int G>
struct CfgQ {
  static constexpr int TSUB = 8 / G;
  static constexpr int BQ = 32 * TSUB;
  static constexpr int CPR = D / 8;
  static constexpr int TBYTES = BK * D * 2;
};

// HOLE: a layout with Gen Images; the block walks its tile list (positions below the
// count of inside FULL tiles need no mask) and masked tiles also hide keys whose
// visibility ends at or before the row.
template <int D, int G, bool HOLE>
__global__ __launch_bounds__(512, 2) void bwd_dq(BwdArgs a) {
  using C = CfgQ<D, G>;
  __shared__ __attribute__((aligned(1024))) char k0[C::TBYTES];
  __shared__ __attribute__((aligned(1024))) char k1[C::TBYTES];
  __shared__ __attribute__((aligned(1024))) char v0[C::TBYTES];
  __shared__ __attribute__((aligned(1024))) char v1[C::TBYTES];

  const int S = a.S, nq = a.nq;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hg = wave % G, tsub = wave / G;
  const int hi = lane >> 5, ln = lane & 31;
  int bg, slot;
  pair_slot(blockIdx.x, a.B * a.Hkv, nq, &bg, &slot);
  const int b = bg / a.Hkv, g = bg % a.Hkv, h = g * G + hg;
  const int qb = nq - 1 - slot;  // query blocks from the last (full rows) to the first
  const int i = S - (nq - qb) * C::BQ + tsub * 32 + ln;
  const bool row_ok = i >= 0;
  const int ic = row_ok ? i : 0;
  const int lim = row_ok ? a.row_limit[(int64_t)b * S + i] : 0;
  const int32_t* cnt = HOLE ? a.tile_count : a.ranges;
  const int kfull = cnt[((int64_t)b * nq + qb) * 2 + 0];
  const int kend = cnt[((int64_t)b * nq + qb) * 2 + 1];
  const int32_t* tlist = HOLE ? a.tiles + ((int64_t)b * nq + qb) * a.nk : nullptr;
  auto tile_at = [&](int t) __attribute__((always_inline)) {
    if constexpr (HOLE)
      return ((const __attribute__((address_space(4))) int32_t*)tlist)[t];  // scalar loads (written before the launch)
    else
      return t;
  };

  const int64_t kvstride = (int64_t)a.Hkv * D * 2;
  const char* kbase = static_cast<const char*>(a.k) + ((int64_t)b * S * a.Hkv + g) * D * 2;
  const char* vbase = static_cast<const char*>(a.v) + ((int64_t)b * S * a.Hkv + g) * D * 2;
  RowDma<D, 2 * D, C::TBYTES / 1024> kvd;
  kvd.init(lane);
  kvd.issue(kbase, kvstride, tile_at(0) * BK, S - 1, k0, wave);
  kvd.issue(vbase, kvstride, tile_at(0) * BK, S - 1, v0, wave);

  // the row's q' and dO as B operands (dims 16kk + 8hi .. +8), its log2(e) lse and delta
  bf16x8 qf[D / 16], of[D / 16];
  const __bf16* qp = static_cast<const __bf16*>(a.q) + (((int64_t)b * S + ic) * a.Hq + h) * D;
  const __bf16* op = static_cast<const __bf16*>(a.dout) + (((int64_t)b * S + ic) * a.Hq + h) * D;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    qf[kk] = *reinterpret_cast<const bf16x8*>(qp + 16 * kk + 8 * hi);
    of[kk] = *reinterpret_cast<const bf16x8*>(op + 16 * kk + 8 * hi);
  }
  const float l2 = a.lse[((int64_t)b * a.Hq + h) * S + ic] * kLog2e;
  const float de = a.delta[((int64_t)b * a.Hq + h) * S + ic];

  f32x16 dq[D / 32];
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) dq[mt] = f32x16{};

  auto step = [&](auto par_tag, auto mask_tag, int t) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par_tag)::value;
    constexpr bool MASKED = decltype(mask_tag)::value;
    const char* const kc = PAR ? k1 : k0;
    const char* const vc = PAR ? v1 : v0;
    char* const kn = PAR ? k0 : k1;
    char* const vn = PAR ? v0 : v1;
    wait_vm();
    __syncthreads();
    if (t + 1 < kend) {
      kvd.issue(kbase, kvstride, tile_at(t + 1) * BK, S - 1, kn, wave);
      kvd.issue(vbase, kvstride, tile_at(t + 1) * BK, S - 1, vn, wave);
    }
    const int tile = tile_at(t);
    // LDS addresses from an opaque copy of the lane id, rebuilt each step (kept live
    // across the loop they would not fit in registers)
    int lo = lane;
    __asm__ volatile("" : "+v"(lo));
    const int lnx = lo & 31, hix = lo >> 5;
    const int kxx = hix ^ swz<C::CPR>(lnx);
    // per 32-key half: S^T = K Q'^T and dP^T = V dO^T (keys x rows, lane = row), then
    // dZ^T = P^T (dP^T - delta) on allowed keys, to bf16 in B-operand order (keys
    // 16KS .. 16KS + 15 of the tile in register order)
    bf16x8 zf[4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f32x16 st = f32x16{}, pt = f32x16{};
      // chunk 2kk + hi of K / V row 32kt + ln sits at (2kk) ^ kxx: the lane's kk = 0 offset
      // XOR 32 kk (the row offset lies above the chunk bits)
      int xr = (32 * kt + lnx) * (2 * D) + kxx * 16;
      __asm__ volatile("" : "+v"(xr));
      auto rd = [&](const char* buf, int kk) __attribute__((always_inline)) {
        return *reinterpret_cast<const bf16x8*>(buf + (xr ^ (32 * kk)));
      };
      // operands of k-step kk + 1 are read while the two MFMAs of k-step kk run
      bf16x8 fk[2], fv[2];
      fk[0] = rd(kc, 0);
      fv[0] = rd(vc, 0);
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const int cur = kk & 1, nxt = cur ^ 1;
        if (kk + 1 < D / 16) {
          fk[nxt] = rd(kc, kk + 1);
          fv[nxt] = rd(vc, kk + 1);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // the two DS reads of kk + 1
        }
        st = mfma(fk[cur], qf[kk], st);
        pt = mfma(fv[cur], of[kk], pt);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);    // then the two MFMAs of kk
      }
      f32x16 pe;
#pragma unroll
      for (int r = 0; r < 16; ++r) pe[r] = __builtin_amdgcn_exp2f(st[r] - l2);
      if constexpr (MASKED) {
        // element r is key tile BK + 32kt + 8(r/4) + 4hi + r%4: allowed below the row's
        // limit and, with Gen Images, when its visibility ends after the row
        const int rem = lim - (tile * BK + 32 * kt + 4 * hix);
        i32x4 vis[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) vis[q4] = i32x4{S, S, S, S};
        if (HOLE) {
          const int* kvp = a.key_vis + (int64_t)b * a.kv_stride + tile * BK + 32 * kt + 4 * hix;
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) vis[q4] = *reinterpret_cast<const i32x4*>(kvp + 8 * q4);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bool ok = 8 * (r >> 2) + (r & 3) < rem && (!HOLE || i < vis[r >> 2][r & 3]);
          pe[r] = ok ? pe[r] : 0.f;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) zf[2 * kt + (r >> 3)][r & 7] = static_cast<__bf16>(pe[r] * (pt[r] - de));
    }
    // dQ^T += K^T dZ^T: A = K^T (dims 32mt .., keys of step KS) gathered from LDS; lane t
    // of 16-lane group G16 points at key 16KS + 8rr + 4(G16 >> 1) + t/4, dims 32mt +
    // 16(G16 & 1) + 4(t & 3). Keys 16KS + r share swz(r) and 4mt + vcl = 4mt ^ vcl, so the
    // address is the lane's (KS = 0, mt = 0) offset XOR 64 mt, plus KS * 16 rows.
    const int g16 = lo >> 4, t16 = lo & 15;
    const int vrow = 4 * (g16 >> 1) + (t16 >> 2);
    const int vclow = 2 * (g16 & 1) + ((t16 & 3) >> 1);
    const int vhalf = 8 * (t16 & 1);
    int tl = vrow * (2 * D) + ((vclow ^ swz<C::CPR>(vrow)) * 16) + vhalf;
    int tu = (vrow + 8) * (2 * D) + ((vclow ^ swz<C::CPR>(vrow + 8)) * 16) + vhalf;
    __asm__ volatile("" : "+v"(tl), "+v"(tu));
    auto trd = [&](int j) __attribute__((always_inline)) {
      const int KS = j / (D / 32), mt = j % (D / 32);
      const char* base = kc + KS * 16 * (2 * D);
      const bf16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + (tl ^ (64 * mt))));
      const bf16x4 up4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + (tu ^ (64 * mt))));
      return __builtin_shufflevector(lo4, up4, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    // the two transposing reads of (KS, mt) + 1 are issued while the MFMA of (KS, mt) runs
    constexpr int NJ = (BK / 16) * (D / 32);
    bf16x8 ka[2];
    ka[0] = trd(0);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int cur = j & 1, nxt = cur ^ 1;
      if (j + 1 < NJ) {
        ka[nxt] = trd(j + 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // the two reads of j + 1
      }
      const int KS = j / (D / 32), mt = j % (D / 32);
      dq[mt] = mfma(ka[cur], zf[KS], dq[mt]);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // then the MFMA of j
    }
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using Full = std::integral_constant<bool, false>;
  using Masked = std::integral_constant<bool, true>;
  // the walk's first tiles need no per-pair mask: every row of the block sees all of their
  // keys and they lie inside the sequence (the list's inside FULL tiles, or tiles below
  // kfull that end by S); an even count of them takes the unmasked step
  const int nf = min(HOLE ? kfull : min(kfull, S / BK), kend) & ~1;
  int t = 0;
  for (; t < nf; t += 2) {
    step(P0{}, Full{}, t);
    step(P1{}, Full{}, t + 1);
  }
  for (; t + 1 < kend; t += 2) {
    step(P0{}, Masked{}, t);
    step(P1{}, Masked{}, t + 1);
  }
  if (t < kend) step(P0{}, Masked{}, t);

  // dQ for the rotated q: scale * sum dZ k; element (mt, r) is dim 32mt + 8(r/4) + 4hi + r%4
  if (row_ok) {
    float* dqo = a.dq + (((int64_t)b * S + i) * a.Hq + h) * D;
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<f32x4*>(dqo + 32 * mt + 8 * j + 4 * hi) =
            f32x4{dq[mt][4 * j] * a.scale, dq[mt][4 * j + 1] * a.scale, dq[mt][4 * j + 2] * a.scale,
                  dq[mt][4 * j + 3] * a.scale};
  }
}

// ====================================================================== launch
// keys [k_begin, k_end) in blocks of CfgKV<D, G, HPS>::KB, each block's steps in n_parts
// ranges (n_parts > 1: partial sums to a.part_dk / a.part_dv)
template <int D, int G, int HPS>
hipError_t launch_kv(BwdArgs a, int k_begin, int k_end, int n_parts, hipStream_t stream) {
  using C = CfgKV<D, G, HPS>;
  a.k_begin = k_begin;
  a.k_end = k_end;
  a.n_parts = n_parts;
  if (n_parts == 1) a.part_dk = a.part_dv = nullptr;
  const int64_t nkb = (k_end - k_begin + C::KB - 1) / C::KB;
  const dim3 grid((unsigned)((int64_t)a.B * a.Hkv * nkb * n_parts));
  if (a.key_vis)
    hipLaunchKernelGGL((bwd_dkdv<D, G, true, HPS>), grid, dim3(512), 0, stream, a);
  else
    hipLaunchKernelGGL((bwd_dkdv<D, G, false, HPS>), grid, dim3(512), 0, stream, a);
  return hipGetLastError();
}

// sums the tail's partial dK and dV over the parts in part order: dk (fp32) and dv (bf16)
// of keys [k_main, S)
__global__ __launch_bounds__(256) void kv_part_sum_kernel(const float* part_dk, const float* part_dv, int parts,
                                                          int64_t n, int64_t per_item, int64_t item_stride,
                                                          int64_t item_off, float* dk, __bf16* dv) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float sk = 0.f, sv = 0.f;
  for (int p = 0; p < parts; ++p) {
    sk += part_dk[p * n + i];
    sv += part_dv[p * n + i];
  }
  const int64_t b = i / per_item, r = i % per_item;
  const int64_t at = b * item_stride + item_off + r;
  dk[at] = sk;
  dv[at] = static_cast<__bf16>(sv);
}

// keys [0, k_main) two heads per step over 128-key blocks (G = 4), the rest with HPS = G,
// their steps in tail_parts ranges whose partial sums are then added (see BwdArgs)
template <int D, int G>
hipError_t launch_kv_plan(const BwdArgs& a, hipStream_t stream) {
  if (a.k_main > 0) {
    const hipError_t e = launch_kv<D, 4, 2>(a, 0, a.k_main, 1, stream);
    if (e != hipSuccess) return e;
  }
  if (a.k_main >= a.S) return hipSuccess;
  const hipError_t e = launch_kv<D, G, G>(a, a.k_main, a.S, a.tail_parts, stream);
  if (e != hipSuccess || a.tail_parts == 1) return e;
  const int64_t per_item = (int64_t)(a.S - a.k_main) * a.Hkv * D;
  const int64_t n = (int64_t)a.B * per_item;
  hipLaunchKernelGGL(kv_part_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a.part_dk,
                     a.part_dv, a.tail_parts, n, per_item, (int64_t)a.S * a.Hkv * D, (int64_t)a.k_main * a.Hkv * D,
                     a.dk, static_cast<__bf16*>(a.dv));
  return hipGetLastError();
}

template <int D, int G>
hipError_t launch_q(const BwdArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)a.B * a.Hkv * a.nq));
  if (a.tiles)
    hipLaunchKernelGGL((bwd_dq<D, G, true>), grid, dim3(512), 0, stream, a);
  else
    hipLaunchKernelGGL((bwd_dq<D, G, false>), grid, dim3(512), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

int bwd_block_k(int group) { return 32 * (8 / group); }

KvPlan kv_plan(int B, int S, int Hkv, int G, int n_cus) {
  KvPlan p;
  if (n_cus <= 0 || S <= 0) return p;
  const int64_t pairs = (int64_t)B * Hkv;
  if (G == 4) {  // two-head blocks only where they fill at least two whole rounds of the CUs
    const int64_t rounds = pairs * (S / CfgKV<128, 4, 2>::KB) / n_cus;
    if (rounds >= 2) p.k_main = (int)(rounds * n_cus / pairs * CfgKV<128, 4, 2>::KB);
  }
  // the rest after two-head blocks, in blocks of 256/G keys: cut their steps into P ranges
  // when that spreads the blocks over fewer rounds per unit of work (by 15% or more). Without
  // a two-head part the blocks are many and the partial sums' traffic costs more than the
  // rounds save (hd1024 in two ranges: 0.371 -> 0.387 ms).
  if (p.k_main == 0) return p;
  const int kb = 32 * (8 / G);
  const int64_t blocks = pairs * ((S - p.k_main + kb - 1) / kb);
  if (blocks <= 0) return p;
  auto cost = [&](int parts) { return (double)((blocks * parts + n_cus - 1) / n_cus) / parts; };
  double best = cost(1);
  for (int parts = 2; parts <= 4; ++parts)
    if (cost(parts) <= 0.85 * best) {
      best = cost(parts);
      p.tail_parts = parts;
    }
  return p;
}

hipError_t launch_bwd_delta(const void* out, const void* dout, float* delta, int B, int S, int Hq, int D,
                            hipStream_t stream) {
  const int64_t threads = (int64_t)B * S * Hq * (D / 8);
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (D == 128)
    hipLaunchKernelGGL((bwd_delta<128>), grid, dim3(256), 0, stream, static_cast<const __bf16*>(out),
                       static_cast<const __bf16*>(dout), delta, B, S, Hq);
  else
    hipLaunchKernelGGL((bwd_delta<64>), grid, dim3(256), 0, stream, static_cast<const __bf16*>(out),
                       static_cast<const __bf16*>(dout), delta, B, S, Hq);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  if (a.D == 128)
    return G == 1 ? launch_kv_plan<128, 1>(a, stream) : G == 2 ? launch_kv_plan<128, 2>(a, stream) : launch_kv_plan<128, 4>(a, stream);
  return G == 1 ? launch_kv_plan<64, 1>(a, stream) : G == 2 ? launch_kv_plan<64, 2>(a, stream) : launch_kv_plan<64, 4>(a, stream);
}

hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  if (a.D == 128) return G == 1 ? launch_q<128, 1>(a, stream) : G == 2 ? launch_q<128, 2>(a, stream) : launch_q<128, 4>(a, stream);
  return G == 1 ? launch_q<64, 1>(a, stream) : G == 2 ? launch_q<64, 2>(a, stream) : launch_q<64, 4>(a, stream);
}

}  // namespace ha
