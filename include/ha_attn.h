/*
 * ha_attn.h -- hybrid-masked joint self-attention for unified text+pixel image
 * transformers, on AMD Instinct MI355X (gfx950).
 *
 * One sequence holds text, condition and generation tokens; each token carries a segment
 * type that fixes which keys its query row may attend to:
 *   HA_SEG_CAUSAL  text, markers, condition and reference tokens: keys j <= i
 *                  (HiDream-O1 atlas page, "How it works"; hidream-o1-p100a model card,
 *                  "What this model is"; HunyuanImage 3.0 digest, "Generalized Causal
 *                  Attention", text rows)
 *   HA_SEG_FULL    HiDream-O1 generation tokens: every key of the sequence (same pages)
 *   HA_SEG_GCA     HunyuanImage 3.0 image tokens: keys j <= i plus every key of their own
 *                  image segment (HunyuanImage 3.0 digest, "Generalized Causal Attention",
 *                  the core rule)
 *   HA_SEG_GEN     a Gen Image of a multi-image HunyuanImage 3.0 training sequence: its
 *                  rows as HA_SEG_GCA, and no token after the segment attends to it, which
 *                  leaves a hole below the diagonal (same digest and section, the
 *                  multi-generation training paragraph and Figure 4(b))
 * Scores use GQA (consecutive groups of n_q_heads / n_kv_heads query heads share one KV
 * head), optional q/k RMSNorm and 1D / generalized 2D / 3-axis interleaved rotary
 * embeddings (hidream-o1-p100a model card, architecture paragraph; HunyuanImage 3.0
 * digest, "Generalized 2D Rotary Position Embedding").
 *
 * Conventions shared by every entry point
 *  - Layouts: q and out are [batch][seq_len][n_q_heads][head_dim]; k and v are
 *    [batch][seq_len][n_kv_heads][head_dim]; all contiguous, token-major, in the dtype of
 *    the descriptor (bf16 or fp32). Device pointers must be 16-byte aligned.
 *  - Ownership: the caller owns every buffer. The library allocates no device memory;
 *    scratch space comes from the caller's workspace. Inputs are never written, except
 *    through the explicit q_out == q_in / k_out == k_in alias of ha_qk_prologue.
 *  - Streams: every launch is asynchronous on the caller's hipStream_t, passed as void*
 *    (NULL = the default stream). No call synchronises, unless the environment variable
 *    HA_DEBUG=1 is set (read at each call), which synchronises and checks for errors after
 *    each launch, and checks rotary positions on the device before they are used: a
 *    position outside [0, n_pos) then fails the call with HA_ERR_INVALID_ARG (without
 *    HA_DEBUG such positions are clamped to that range; the pages' contract convention
 *    is to reject contract errors, hidream-o1-p100a model card, "Serving (HTTP)").
 *  - Errors: every argument is validated on the host before any HIP call (HA_DEBUG's
 *    position check aside). A bad call returns a nonzero ha_status, sets the thread's
 *    ha_last_error() text, and touches neither the device nor the stream. A failed launch
 *    returns HA_ERR_HIP with the HIP error text. No C++ exception crosses this interface.
 *    The library keeps no state between calls apart from that error text and, for
 *    ha_attn_fwd_static alone, its per-device scratch array and that array's looked-up
 *    device address (see there).
 *  - Empty work (batch == 0 or seq_len == 0) is valid and launches nothing.
 */
#ifndef HA_ATTN_H
#define HA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HA_ABI_VERSION 5
#define HA_MAX_SEGMENTS 64      /* segments per batch item */
#define HA_MAX_SEQ_LEN (1 << 22)

typedef enum {
  HA_OK = 0,
  HA_ERR_INVALID_ARG = 1,   /* null pointer, bad count, bad enum, bad scale/eps */
  HA_ERR_UNSUPPORTED = 2,   /* valid but not implemented (head_dim, head ratio, sizes) */
  HA_ERR_SEGMENTS = 3,      /* segment table does not tile [0, seq_len) */
  HA_ERR_ALIGNMENT = 4,     /* device pointer not 16-byte (weights: 4-byte) aligned */
  HA_ERR_WORKSPACE = 5,     /* workspace missing, too small or not 256-byte aligned */
  HA_ERR_HIP = 6            /* a HIP launch or runtime call failed */
} ha_status;

typedef enum { HA_SEG_CAUSAL = 0, HA_SEG_FULL = 1, HA_SEG_GCA = 2, HA_SEG_GEN = 3 } ha_seg_kind;
typedef enum { HA_DTYPE_BF16 = 0, HA_DTYPE_F32 = 1 } ha_dtype;
typedef enum { HA_ROPE_NONE = 0, HA_ROPE_1D = 1, HA_ROPE_2D = 2, HA_ROPE_MROPE = 3 } ha_rope_kind;
typedef enum { HA_TILE_SKIP = 0, HA_TILE_FULL = 1, HA_TILE_PARTIAL = 2 } ha_tile_label;

/* One segment of one batch item: tokens [start, start + length) of kind ha_seg_kind.
 * A batch item's segments must be listed in order, contiguous from 0, with positive
 * lengths summing to seq_len. Adjacent image segments are distinct images. */
typedef struct {
  int32_t start;
  int32_t length;
  int32_t kind;
} ha_segment;

typedef struct {
  int32_t batch;            /* >= 0 */
  int32_t seq_len;          /* >= 0, <= HA_MAX_SEQ_LEN */
  int32_t n_q_heads;        /* >= 1 */
  int32_t n_kv_heads;       /* >= 1, divides n_q_heads; n_q_heads / n_kv_heads in {1,2,4,8} */
  int32_t head_dim;         /* 64 or 128 */
  int32_t dtype;            /* ha_dtype of q, k, v, out */
  const ha_segment* segments; /* HOST memory, [batch][n_segments] */
  int32_t n_segments;       /* 1 .. HA_MAX_SEGMENTS (per batch item) */
  float scale;              /* softmax scale; 0 means 1 / sqrt(head_dim) */
  int32_t q_prescaled;      /* ha_attn_fwd_planned only: 1 when q already carries the factor
                               scale * log2(e) (ha_qk_prologue with q_out_scale set to
                               ha_q_prescale(desc)), 0 for plain q */
  int32_t split_parts;      /* split plan of the bf16 forward (see ha_attn_fwd): 0 lets the
                               planner decide, 1 never splits, P in [2, 64] splits every
                               query block into P parts */
  int32_t plan_cus;         /* CUs the work is balanced over (the forward's split plan,
                               the backward's dK/dV launches): 0 means the current
                               device's count, n > 0 plans for n CUs */
} ha_attn_desc;

/* q/k prologue: RMSNorm over head_dim (y = x / sqrt(mean(x^2) + eps) * w, before the
 * rotation; model card "q/k RMSNorm"), then the rotary embedding. Pair i of a head is
 * (x[i], x[i + head_dim/2]) and is rotated by angle positions[axis(i)] * theta^(-2i/d):
 *   HA_ROPE_1D     axis(i) = 0                      (positions [B][S][1])
 *   HA_ROPE_2D     axis(i) = i mod 2, 0 = x (column), 1 = y (row)   ([B][S][2])
 *   HA_ROPE_MROPE  pairs dealt to axes 0,1,2 (T, H, W) in turn, each axis leaving the
 *                  rotation once it holds mrope_sections[axis] pairs ([B][S][3]);
 *                  [24,20,20] gives i mod 3 for i < 60 and T for 60..63
 *   HA_ROPE_NONE   no rotation (positions and cos_sin may be NULL)
 * Positions must lie in [0, n_pos): HA_DEBUG=1 checks them on the device and fails the call
 * otherwise; without it, out-of-range positions are clamped to that range. */
typedef struct {
  int32_t rope_kind;            /* ha_rope_kind */
  int32_t mrope_sections[3];    /* HA_ROPE_MROPE only; non-negative, sum head_dim / 2 */
  const int32_t* positions;     /* DEVICE [batch][seq_len][n_axes] */
  const float* cos_sin;         /* DEVICE [n_pos][head_dim/2][2] from ha_rope_table_fill */
  int32_t n_pos;                /* rows of cos_sin */
  const float* q_norm_weight;   /* DEVICE fp32 [head_dim], or NULL for no RMSNorm */
  const float* k_norm_weight;   /* DEVICE fp32 [head_dim]; NULL exactly when q's is */
  float eps;                    /* RMSNorm epsilon, >= 0 */
  float q_out_scale;            /* q outputs are multiplied by this before rounding; 0 means 1 */
} ha_prologue_desc;

/* HA_ABI_VERSION of the built library. */
int ha_abi_version(void);

/* Text of the calling thread's last error ("" if none). Never NULL. */
const char* ha_last_error(void);

/* Fill host_out [n_pos][head_dim/2][2] with (cos, sin) of p * theta^(-2i/head_dim) for
 * p in [0, n_pos), i in [0, head_dim/2), computed in double and rounded to float.
 * Host-only; theta > 1, head_dim in {64, 128}, n_pos >= 1. */
ha_status ha_rope_table_fill(double theta, int32_t head_dim, int32_t n_pos, float* host_out);

/* The factor scale * log2(e) that a prescaled q carries (see ha_attn_desc.q_prescaled).
 * Returns 0 for an invalid descriptor. */
float ha_q_prescale(const ha_attn_desc* desc);

/* Tile grid used by the attention kernel for this descriptor: block_q query tokens by
 * block_k keys, n_q_blocks x n_k_blocks tiles. Key tiles start at index 0 (the last one
 * ragged). Query blocks are aligned to the end of the sequence: block qb covers rows
 * [S - (n_q_blocks - qb) * block_q, S - (n_q_blocks - qb - 1) * block_q) clipped at 0, so
 * the first block is the ragged one and the generation tokens that end the pages' layouts
 * fill whole blocks. */
ha_status ha_tile_shape(const ha_attn_desc* desc, int32_t* block_q, int32_t* block_k,
                        int32_t* n_q_blocks, int32_t* n_k_blocks);

/* Segment-table tile classifier. Every query row i may attend to a key prefix
 * [0, lim(i)): causal rows lim = i + 1, full rows lim = seq_len, image (GCA and Gen)
 * rows lim = end of their segment; Gen Images then cut holes into the prefixes of the
 * rows after them. Writes, on the stream:
 *   row_limit [batch][seq_len] int32        lim(i), before any hole      (may be NULL)
 *   ranges    [batch][n_q_blocks][2] int32  (kfull, kend) from the row limits: without
 *                                           Gen Images tiles [0, kfull) are FULL,
 *                                           [kfull, kend) PARTIAL, the rest SKIP
 *   labels    [batch][n_q_blocks][n_k_blocks] uint8 ha_tile_label, holes included
 *                                                                         (may be NULL)
 * Tiles follow ha_tile_shape's grid (query blocks end-aligned).
 * Over the valid part of a tile (rows and keys in [0, seq_len)): SKIP = no allowed pair,
 * FULL = all allowed, PARTIAL = otherwise. All DEVICE pointers, 4-byte aligned
 * (labels: any alignment). ranges may be NULL only if another output is requested. */
ha_status ha_classify_tiles(const ha_attn_desc* desc, uint8_t* labels, int32_t* ranges,
                            int32_t* row_limit, void* stream);

/* Fused q/k RMSNorm + rotary embedding (see ha_prologue_desc). Reads q_in, k_in and
 * writes q_out, k_out (same layouts and dtype; out may alias in exactly). */
ha_status ha_qk_prologue(const ha_attn_desc* desc, const ha_prologue_desc* pro,
                         const void* q_in, const void* k_in, void* q_out, void* k_out,
                         void* stream);

/* Workspace bytes ha_attn_fwd needs: row limits, tile ranges, and the rotated q and k
 * when pro is not NULL; with HA_SEG_GEN segments also per-key visibility and per query
 * block tile lists; with a split plan (below) its work item table and fp32 partial
 * results. The plan depends on the CU count (desc->plan_cus, else the current device's),
 * so call this with the device current that will run the forward. */
size_t ha_attn_workspace_bytes(const ha_attn_desc* desc, const ha_prologue_desc* pro);

/* Attention on prepared inputs: q and k already normalised and rotated (q optionally
 * prescaled, see ha_attn_desc.q_prescaled), row_limit and ranges from ha_classify_tiles
 * for the same descriptor (so the tile plan can be reused across layers and denoising
 * steps). out = softmax(scale * q k^T, masked) v per query head, fp32 accumulation, P
 * rounded to the input dtype for the second product. Layouts with HA_SEG_GEN segments
 * need more of the plan than row_limit and ranges: they return HA_ERR_UNSUPPORTED here
 * (and in ha_attn_fwd_planned_from); ha_attn_fwd, ha_attn_fwd_lse and ha_attn_bwd take
 * them. One work item per query block: the split plan of ha_attn_fwd (below) needs its
 * workspace. */
ha_status ha_attn_fwd_planned(const ha_attn_desc* desc, const void* q, const void* k,
                              const void* v, const int32_t* row_limit, const int32_t* ranges,
                              void* out, void* stream);

/* The whole path: classifier, prologue (skipped when pro is NULL: q, k are then used as
 * given), attention. With a prologue, the q it writes to the workspace is prescaled (its
 * q_out_scale is ignored) and desc->q_prescaled is ignored. workspace: DEVICE, 256-byte
 * aligned, >= ha_attn_workspace_bytes.
 *
 * Split plan (bf16): where the heaviest query blocks would leave the CUs partly idle in
 * their last round (e.g. the HunyuanImage 3.0 interleave, or fewer blocks than CUs), the
 * host decides, from the segment table, to split some blocks' key tiles into parts that
 * run as separate work items, and a merge kernel combines them (the merge rounds
 * differently from one work item: results agree within bf16 rounding, not bit for bit,
 * with ha_attn_fwd_planned). A kernel builds the work item table in the workspace from
 * the classifier's per-block tile counts (longest first on each XCD), so the call copies
 * nothing from the host and allocates nothing. The plan covers at most 1024 work items per
 * XCD before splitting; larger problems run one work item per query block. A workspace
 * smaller than ha_attn_workspace_bytes but large enough without the plan runs without
 * it. desc->split_parts and desc->plan_cus override the planner (for tests). */
ha_status ha_attn_fwd(const ha_attn_desc* desc, const ha_prologue_desc* pro, const void* q,
                      const void* k, const void* v, void* out, void* workspace,
                      size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- step-invariant prefix
 * Causal rows see only keys at or before themselves (HiDream-O1 atlas page, "How it works":
 * text and condition tokens are causal). So a causal prefix of the sequence (the text
 * tokens and markers at its front) never sees the generation tokens after it, and its
 * outputs and its k, v stay the same across the denoising steps of one image (model card,
 * "What this model is": the same layout for every step). This reuse follows from the mask;
 * the pages do not describe it. A caller that keeps the previous step's rotated q, k and the
 * output of such a prefix [0, p) recomputes only what follows it: */

/* ha_qk_prologue on tokens [token_begin, seq_len) of every batch item; the rest of q_out,
 * k_out is not touched. 0 <= token_begin <= seq_len. */
ha_status ha_qk_prologue_from(const ha_attn_desc* desc, const ha_prologue_desc* pro,
                              const void* q_in, const void* k_in, void* q_out, void* k_out,
                              int32_t token_begin, void* stream);

/* ha_attn_fwd_planned for the query rows [row_begin, seq_len) only: the query blocks that
 * hold them are computed (from all of q, k, v: the prefix's q, k, v must be in place), and
 * out rows below row_begin are not written. 0 <= row_begin <= seq_len, and no row below
 * row_begin may attend to a key at or after it (so the kept rows are exact): a full
 * segment that starts below row_begin < seq_len, or an image segment that row_begin cuts,
 * fails the call with HA_ERR_INVALID_ARG. A causal prefix qualifies. */
ha_status ha_attn_fwd_planned_from(const ha_attn_desc* desc, const void* q, const void* k,
                                   const void* v, const int32_t* row_limit, const int32_t* ranges,
                                   void* out, int32_t row_begin, void* stream);

/* ---------------------------------------------------------------- QKV projection
 * The step before the path: each backbone layer projects its normalised hidden states to
 * q, k and v by one linear map (hidream-o1-p100a model card, "What this model is": hidden
 * 4096, GQA 32/8, head dim 128, q/k RMSNorm, mRoPE). This call computes the projection on
 * the matrix cores and applies the prologue (see ha_qk_prologue) to q and k in the same
 * kernel, before anything is written, so q, k and v reach HBM once, in bf16, in the
 * layouts ha_attn_fwd_planned reads:
 *   x      DEVICE bf16 [batch][seq_len][hidden], hidden a positive multiple of 64
 *   w_qkv  DEVICE bf16 [(n_q_heads + 2 n_kv_heads) * 128][hidden]: the linear layer's
 *          weight, rows the q heads, then the k heads, then the v heads; y = x w_qkv^T,
 *          no bias, accumulated in fp32 and not rounded before the prologue
 *   q_out  [batch][seq_len][n_q_heads][128], k_out and v_out [batch][seq_len][n_kv_heads][128]
 * pro may be NULL (a plain projection); its q_out_scale multiplies q (0 means 1). bf16 and
 * head_dim 128 only (else HA_ERR_UNSUPPORTED). The segment table is not consulted. */
ha_status ha_qkv_prologue(const ha_attn_desc* desc, const ha_prologue_desc* pro, const void* x,
                          int32_t hidden, const void* w_qkv, void* q_out, void* k_out, void* v_out,
                          void* stream);

/* ---------------------------------------------------------------- training
 * The pages train these models end to end (HiDream-O1 atlas page, "How it works";
 * HunyuanImage 3.0 digest, training stages); the backward below is the derivative of the
 * forward above (the pages print no backward formulas). bf16 only, n_q_heads / n_kv_heads
 * in {1, 2, 4}; fp32 descriptors and groups of 8 return HA_ERR_UNSUPPORTED. */

/* ha_attn_fwd, also writing the row log-sum-exp the backward needs: lse, DEVICE fp32
 * [batch][n_q_heads][seq_len], the natural log of sum_j exp(scale q_i . k_j) over the keys
 * row i attends (q, k after the prologue). The scores are those ha_attn_bwd rebuilds: with
 * q' = scale log2(e) q rounded to bf16, which the prologue writes, or which this call
 * forms from q itself when pro is NULL and q is not prescaled; so the lse and the
 * backward's probabilities agree to fp32 rounding. Same workspace as ha_attn_fwd. */
ha_status ha_attn_fwd_lse(const ha_attn_desc* desc, const ha_prologue_desc* pro, const void* q,
                          const void* k, const void* v, void* out, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Workspace bytes ha_attn_bwd needs: row limits, tile ranges, the rebuilt prologue
 * outputs, per-row dout . out, fp32 gradients of the rotated q and k, with RMSNorm
 * per-token weight-gradient partials, and with HA_SEG_GEN segments the key visibility and
 * tile lists. */
size_t ha_attn_bwd_workspace_bytes(const ha_attn_desc* desc, const ha_prologue_desc* pro);

/* Gradients for the output gradient dout (same layout as out): dq, dk, dv with respect
 * to ha_attn_fwd_lse's inputs q, k, v (same layouts; all bf16, DEVICE, 16-byte aligned);
 * with RMSNorm in pro, dw_q and dw_k (DEVICE fp32 [head_dim], overwritten) with respect to
 * the norm weights, else they must be NULL. out and lse are the forward's for the same
 * desc, pro and inputs. desc->q_prescaled must be 0 (q is the path's input). The prologue
 * is recomputed in the workspace (DEVICE, 256-byte aligned, >= ha_attn_bwd_workspace_bytes);
 * nothing is allocated. Gradients accumulate in fp32; dq, dk, dv are rounded to bf16. */
ha_status ha_attn_bwd(const ha_attn_desc* desc, const ha_prologue_desc* pro, const void* q,
                      const void* k, const void* v, const void* out, const float* lse,
                      const void* dout, void* dq, void* dk, void* dv, float* dw_q, float* dw_k,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- allocation-free forward
 * For callers that cannot allocate: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc. ha_attn_fwd with pro == NULL (q, k already normalised and
 * rotated; plain or prescaled q as desc->q_prescaled says, like ha_attn_fwd_planned), but
 * its scratch (row limits, tile ranges, Gen Image plan, split plan table and partial
 * results) lives in a device array of the library, HA_STATIC_SCRATCH_BYTES per GPU, held
 * from the library's first use on that GPU until the process ends. The call allocates
 * nothing and calls no allocating routine. A problem whose scratch exceeds the array (with
 * the split plan if it fits, else without it) fails with HA_ERR_WORKSPACE before any launch.
 * Every call on a GPU shares that GPU's array and overwrites what it reads before reading
 * it; calls that overlap on one GPU (two streams, two threads) race and must be ordered by
 * the caller. Results equal ha_attn_fwd's bit for bit. */
#define HA_STATIC_SCRATCH_BYTES (16u << 20)
ha_status ha_attn_fwd_static(const ha_attn_desc* desc, const void* q, const void* k, const void* v,
                             void* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HA_ATTN_H */
