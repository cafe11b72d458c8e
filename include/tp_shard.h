/*
 * tp_shard.h -- C ABI of libtpshard: one tensor-parallel (TP) rank's share of a
 * Megatron-style Transformer layer on an AMD MI355X (gfx950).
 *
 * Pages this interface follows (cited by title and section):
 *   [L11] grasp.study Lesson 11, "张量并行线性层分片与前反向通信量计算"
 *         (tensor-parallel linear sharding and fwd/bwd communication volume)
 *   [LP]  cnblogs "ラブパラ" (survey of parallelisms)
 *   [HJ]  hjcheng0602.cn "tensorparallel/tp"
 *   [TP1] "Tensor Parallelism张量并行（一）"
 *
 * Notation ([L11] section 1; [LP] O.I): T = b*s tokens of a microbatch, hidden
 * size h, MLP intermediate size h_ffn, TP degree t, bytes per element delta;
 * per-rank intermediate width f (= h_ffn / t when t divides it; in general
 * tp_mlp_shard_cols), q local query heads and kv local KV heads of width d
 * (= n_q / t and n_kv / t when t divides them; in general tp_attn_shard_heads).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are dense and row-major; tokens are rows (row r = beta*s + sigma).
 *    Weights are stored [in, out] so the layer computes X W (the semantic
 *    orientation of [L11] section 1).
 *  - All tensor pointers are DEVICE pointers owned by the caller, 16-byte
 *    aligned.  A tensor with no elements may be passed as NULL.  The library
 *    never allocates or frees device memory; it keeps none of its own except
 *    the fixed scratch array of tp_attn_shard_bwd_noalloc.  Outputs may not
 *    alias inputs.
 *  - Process-wide inputs, the only state kept between calls (the environment
 *    is never read):
 *      * the launch options of tp_set_options (tile shape, splits), which
 *        change how work is divided, never what is computed beyond rounding
 *        order; default TP_TILE_AUTO with splits on;
 *      * the profiling hook of tp_profile_arm (events only, no results).
 *    Both are safe to set and read from several threads; a call made while
 *    another thread changes the options uses either the old or the new ones.
 *  - Storage type: TP_F32 means every activation, weight and bias is fp32;
 *    TP_BF16 means they are bf16 (products accumulate in fp32).  Weight and
 *    bias gradients (dW*, db*) are always fp32.
 *  - For TP_BF16 the sizes h, h_ffn, (q + 2 kv) d and q d must be multiples of
 *    8; for TP_F32 multiples of 4 (vector width of 16 bytes).
 *  - Every launch is asynchronous on `stream` (a hipStream_t passed as void*;
 *    NULL is the default stream).  Arguments are validated before any launch:
 *    on a negative return nothing was enqueued.  Nothing is printed and no
 *    C++ exception crosses the ABI.
 *  - Calls on one stream run in order; the library adds no synchronisation.
 */
#ifndef TP_SHARD_H
#define TP_SHARD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element storage type of activations and weights (delta = 4 or 2 bytes). */
typedef enum { TP_F32 = 0, TP_BF16 = 1 } tp_dtype;

/* MLP activation: exact-erf GeLU on (X W1 + b1), or SwiGLU SiLU(X Wg) * (X Wu). */
typedef enum { TP_GELU = 0, TP_SWIGLU = 1 } tp_act;

/* Status codes. */
enum {
  TP_OK = 0,
  TP_EINVAL = -1,       /* NULL for a required non-empty tensor, size < 0, t < 1, rank >= t, p outside [0,1) */
  TP_ENOTDIV = -2,      /* a split the shard rules do not cover (see tp_attn_shard_heads; rows % t for the reduce-scatter) */
  TP_EDTYPE = -3,       /* unknown dtype/activation, or a combination not provided (attention in fp32) */
  TP_EALIGN = -4,       /* a pointer is not 16-byte aligned or a width is not a multiple of the vector width */
  TP_EHIP = -5,         /* the HIP runtime reported an error when enqueuing a kernel */
  TP_EUNSUPPORTED = -6, /* a size the kernels do not implement (head width other than 64 or 128, t > 64,
                           an attention shard with s >= 2^24 or a QKV row of 2^24 bytes or more) */
  TP_ENOSCRATCH = -7    /* tp_attn_shard_bwd_noalloc: the problem needs more than the fixed scratch array */
};

/* Tile shape of the matrix-core GEMMs (tp_set_options). */
enum {
  TP_TILE_AUTO = 0,   /* chosen per launch from the tile count (the default) */
  TP_TILE_LARGE = 1,  /* 256 x 256 (256 x 128 with two B operands), eight waves */
  TP_TILE_SMALL = 2,  /* 128 x 128 (128 x 64), four waves */
  TP_TILE_TINY = 3    /* 64 x 64 for single-B launches, else as TP_TILE_SMALL */
};

/* One rank's MLP shard. */
typedef struct {
  int64_t tokens;   /* T = b*s */
  int64_t h;        /* hidden size */
  int64_t h_ffn;    /* full intermediate size; this rank holds f columns (tp_mlp_shard_cols) */
  int32_t t;        /* TP degree (1 = unsharded layer) */
  int32_t rank;     /* which slice this shard is, 0 <= rank < t (informational for the MLP) */
  int32_t dtype;    /* tp_dtype */
  int32_t act;      /* tp_act */
} tp_mlp_desc;

/* One rank's attention shard (forward and backward). */
typedef struct {
  int64_t b, s, h;  /* sequences, sequence length, hidden size; T = b*s */
  int32_t n_q;      /* query heads of the whole layer */
  int32_t n_kv;     /* key/value heads of the whole layer (GQA when < n_q) */
  int32_t d;        /* head width */
  int32_t t;        /* TP degree */
  int32_t rank;     /* 0 <= rank < t */
  int32_t dtype;    /* tp_dtype; only TP_BF16 is provided */
  int32_t causal;   /* 1: key position <= query position; 0: full attention */
} tp_attn_desc;

/* All-reduce accounting of one layer ([L11] section 5; [TP1] communication cost). */
typedef struct {
  int32_t n_allreduce_fwd;            /* 2: after the attention and the MLP output projections */
  int32_t n_allreduce_bwd;            /* 2: at the MLP and the attention inputs */
  uint64_t payload_bytes;             /* logical size of one all-reduce: tokens*h*delta */
  double ring_bytes_per_rank;         /* bytes one rank sends in a ring all-reduce: 2(t-1)/t * payload */
  uint64_t layer_payload_bytes;       /* 4 * payload_bytes */
  double layer_ring_bytes_per_rank;   /* 4 * ring_bytes_per_rank */
} tp_comm;

/*
 * tp_mlp_shard_cols -- the intermediate columns a rank owns (host only).
 * ([L11] section 2 for the even split; [TP1], GQA paragraph: a size that t
 * does not divide needs an uneven split.)
 * The h_ffn columns are cut into contiguous blocks of the storage vector (8
 * bf16 or 4 fp32 columns) dealt out in rank order as evenly as whole blocks
 * allow: with u = h_ffn / vec blocks, rank i gets u / t blocks, plus one if
 * i < u % t (a rank may get none; its partials are then zero).  f_i and col0
 * are this rank's width and first column; f_i = h_ffn / t when t * vec
 * divides h_ffn.  Every MLP entry point uses this split for desc->rank.
 * Errors: TP_EDTYPE, TP_EINVAL (NULL output, h_ffn < 0, rank outside
 * [0, t)), TP_EALIGN (h_ffn not a multiple of the vector width).
 */
int tp_mlp_shard_cols(int64_t h_ffn, int32_t t, int32_t rank, int32_t dtype, int64_t* f_i, int64_t* col0);

/*
 * tp_attn_shard_heads -- the heads a rank owns (host only).
 * ([L11] section 4 and [LP] I.III: a rank holds whole GQA groups; [TP1], GQA
 * paragraph: uneven split when the count does not divide; [LP] III.III: when
 * the split cannot be complete, several ranks share one KV projection, a
 * parameter replica.)
 *   n_kv >= t: the n_kv groups are dealt out in rank order, rank i taking
 *              n_kv / t of them plus one if i < n_kv % t, with all their
 *              n_q / n_kv query heads each;
 *   n_kv <  t: KV head g is replicated on the r = t / n_kv ranks g*r ..
 *              g*r + r - 1, which take (n_q / n_kv) / r of its query heads each
 *              (needs t % n_kv == 0 and (n_q / n_kv) % r == 0).
 * q_i, kv_i: this rank's query / KV head counts; q0, kv0: the first of each.
 * With replicated KV heads the K and V column blocks of tp_attn_shard_bwd's
 * dWqkv_i are this rank's share of that replica's gradient: the ranks that
 * hold the same KV head add them.  Every attention entry point uses this
 * split for desc->rank.
 * Errors: TP_EINVAL (NULL output, counts < 1, rank outside [0, t)),
 * TP_ENOTDIV (n_q % n_kv != 0, or a replication the rule above does not cover).
 */
int tp_attn_shard_heads(int32_t n_q, int32_t n_kv, int32_t t, int32_t rank, int32_t* q_i, int32_t* kv_i,
                        int32_t* q0, int32_t* kv0);

/*
 * tp_mlp_shard_fwd -- forward of one rank's MLP shard
 * ([L11] sections 2-3; [TP1] column split and "MLP and attention"; [HJ] TP forward).
 *
 * Column-parallel GEMM with the activation fused in its epilogue, then the
 * row-parallel GEMM that yields the partial Z_i (output bias NOT added: it is
 * added once after the sum, see tp_sum_partials).
 *   GeLU:   A_i = X W1_i + b1_i;  H_i = GeLU(A_i)
 *   SwiGLU: G_i = X W1_i;  U_i = X Wu_i;  H_i = SiLU(G_i) * U_i
 *   Z_i = H_i W2_i
 * Arguments (T = tokens, f = this rank's width, tp_mlp_shard_cols):
 *   X     [T, h]   replicated input
 *   W1_i  [h, f]   first-layer columns of this rank (the gate for SwiGLU)
 *   Wu_i  [h, f]   SwiGLU up-projection columns; must be NULL for GeLU
 *   b1_i  [f]      GeLU first-layer bias slice, or NULL; must be NULL for SwiGLU
 *   W2_i  [f, h]   second-layer rows of this rank
 *   saved_i        out: GeLU A_i [T, f]; SwiGLU G_i then U_i, two [T, f] blocks
 *   H_i   [T, f]   out: activation
 *   Z_i   [T, h]   out: partial output of this rank.  Its memory is also
 *                  scratch for the column GEMM (fp32 partial tiles when that
 *                  GEMM's last round of tiles is split over K) before the row
 *                  GEMM writes it, so it must not overlap any other argument.
 */
int tp_mlp_shard_fwd(const tp_mlp_desc* desc, const void* X, const void* W1_i, const void* Wu_i,
                     const void* b1_i, const void* W2_i, void* saved_i, void* H_i, void* Z_i,
                     void* stream);

/*
 * tp_mlp_shard_bwd -- backward of one rank's MLP shard
 * ([L11] sections 2-3; [TP1] operator f; [HJ] single-card and TP backward).
 *
 *   dY    = dOut * keep / (1 - p)          (dropout backward; keep as in tp_sum_partials)
 *   db2   = sum over tokens of dY          (output-bias gradient; replicated)
 *   dW2_i = H_i^T dY;  dH_i = dY W2_i^T
 *   GeLU:   dA_i = dH_i * GeLU'(A_i);  db1_i = sum over tokens of dA_i
 *           dW1_i = X^T dA_i;  dX_i = dA_i W1_i^T
 *   SwiGLU: dU_i = dH_i * SiLU(G_i);  dG_i = dH_i * U_i * SiLU'(G_i)
 *           dWg_i = X^T dG_i;  dWu_i = X^T dU_i;  dX_i = dG_i Wg_i^T + dU_i Wu_i^T
 * dX_i is this rank's partial input gradient; the backward all-reduce
 * (tp_sum_partials with no bias and p = 0) sums it over ranks.
 * Arguments:
 *   dOut  [T, h]        gradient of the layer output (replicated)
 *   p_drop, seed        the forward's dropout probability and seed
 *   X, W1_i, Wu_i, W2_i as in tp_mlp_shard_fwd (Wu_i NULL for GeLU)
 *   saved_i, H_i        as written by tp_mlp_shard_fwd
 *   dY    [T, h]        out, act dtype.  May be NULL when p_drop == 0; dOut is then used as dY.
 *   db2   [h] fp32      out, or NULL to skip
 *   dA_i                out, act dtype: GeLU dA_i [T, f]; SwiGLU dG_i then dU_i, two [T, f] blocks
 *   dW1_i fp32          out: GeLU dW1_i [h, f]; SwiGLU dWg_i then dWu_i, two [h, f] blocks
 *   db1_i [f] fp32      out for GeLU, or NULL to skip; must be NULL for SwiGLU
 *   dW2_i [f, h] fp32   out
 *   dX_i  [T, h]        out, act dtype: partial input gradient
 */
int tp_mlp_shard_bwd(const tp_mlp_desc* desc, const void* dOut, float p_drop, uint64_t seed,
                     const void* X, const void* W1_i, const void* Wu_i, const void* W2_i,
                     const void* saved_i, const void* H_i, void* dY, float* db2, void* dA_i,
                     float* dW1_i, float* db1_i, float* dW2_i, void* dX_i, void* stream);

/*
 * tp_attn_shard_fwd -- forward of one rank's attention shard
 * ([L11] section 4; [LP] I.III; [HJ] Attention, single-card forward).
 *
 *   QKV_i = X Wqkv_i, columns [Q heads (q*d) | K heads (kv*d) | V heads (kv*d)], head-major
 *   per sequence and local query head j (KV head j / (q/kv)):
 *     O = softmax(Q K^T / sqrt(d) + mask) V, mask = -inf where key > query (causal)
 *   Z_i = O_i Wo_i   (partial; summed over ranks by tp_sum_partials)
 * Arguments:
 *   X      [T, h]              replicated input, bf16
 *   Wqkv_i [h, (q+2kv) d]      this rank's QKV column shard, bf16
 *   Wo_i   [q d, h]            this rank's output-projection rows, bf16
 *   QKV_i  [T, (q+2kv) d]      out, bf16 (also the attention's input)
 *   O_i    [T, q d]            out, bf16, heads concatenated head-major
 *   lse_i  [b, q, s] fp32      out, natural-log sum of exp of the scaled masked scores per row, or NULL
 *   Z_i    [T, h]              out, bf16 partial.  Its memory is also scratch
 *                              for the attention kernel (softmax state of split
 *                              causal query blocks) before the output
 *                              projection writes it, so it must not overlap any
 *                              other argument.
 * Head widths 64 and 128 are provided.
 */
int tp_attn_shard_fwd(const tp_attn_desc* desc, const void* X, const void* Wqkv_i, const void* Wo_i,
                      void* QKV_i, void* O_i, float* lse_i, void* Z_i, void* stream);

/*
 * tp_attn_shard_bwd -- backward of one rank's attention shard
 * ([HJ] Attention, single-card backward; [LP] I.O on recomputing the scores;
 * [TP1] operators f and g and the attention sublayer's communication).
 *
 *   dWo_i = O_i^T dZ;   dO_i = dZ Wo_i^T
 *   per sequence and local query head j (KV head g = j / (q/kv)), c = 1/sqrt(d),
 *   P = softmax(c Q K^T + mask) recomputed from lse_i:
 *     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - rowsum(dO * O)),
 *     dQ = c dS K,  dK = c dS^T Q   (dK, dV summed over the heads of the group)
 *   dQKV_i = [dQ heads | dK heads | dV heads] (the layout of QKV_i)
 *   dWqkv_i = X^T dQKV_i;   dX_i = dQKV_i Wqkv_i^T
 * dZ is the gradient of the attention sublayer's output, the same on every
 * rank; dX_i is this rank's partial input gradient, summed over ranks by
 * tp_sum_partials (no bias, p = 0).
 * Arguments:
 *   dZ      [T, h]             gradient of the sublayer output (replicated), bf16
 *   X, Wqkv_i, Wo_i            as in tp_attn_shard_fwd
 *   QKV_i, O_i, lse_i          as written by tp_attn_shard_fwd (lse_i required)
 *   dO_i    [T, q d]           out, bf16: gradient of O_i
 *   stats_i [b, q, s, 2] fp32  scratch: per row {lse * log2(e), rowsum(dO * O)}
 *   dQKV_i  [T, (q+2kv) d]     out, bf16
 *   dWqkv_i [h, (q+2kv) d] fp32 out.  Its memory is also scratch for the
 *                          dK/dV kernel (fp32 halves of the split causal key
 *                          blocks, then the dS tiles that do not fit in
 *                          dX_i's) before the last GEMM writes it, so it
 *                          must not overlap any other argument.
 *   dWo_i   [q d, h] fp32      out
 *   dX_i    [T, h]             out, bf16 partial input gradient.  Its memory is
 *                              also scratch before the last GEMM writes it:
 *                              causal, the bf16 dS tiles (2 KiB per 32 x 32
 *                              query x key tile on or below the diagonal)
 *                              that dK/dV hands to dQ when they fit here and
 *                              in dWqkv_i's memory, else the fp32 halves of
 *                              dQ's split causal query blocks; so it must not
 *                              overlap any other argument.
 * Same descriptor and conditions as tp_attn_shard_fwd.  The result does not
 * depend on the order in which work-groups run (no atomics).
 */
int tp_attn_shard_bwd(const tp_attn_desc* desc, const void* dZ, const void* X, const void* Wqkv_i,
                      const void* Wo_i, const void* QKV_i, const void* O_i, const float* lse_i,
                      void* dO_i, float* stats_i, void* dQKV_i, float* dWqkv_i, float* dWo_i,
                      void* dX_i, void* stream);

/*
 * tp_attn_shard_bwd_noalloc -- tp_attn_shard_bwd for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same kernels and results, bit for
 * bit, with the per-row statistics (stats_i) kept in a device array of the
 * library instead of a caller buffer.  The caller still passes every input
 * and output (dWqkv_i and dX_i keep their scratch role).
 *   Limit: 2 * b * q * s floats of statistics, at most 2^20 (4 MiB; b * q * s
 *   <= 524288 local query rows); larger problems return TP_ENOSCRATCH
 *   before anything is enqueued.
 *   The array is per GPU: the call uses the copy of the device current on
 *   the calling thread, which must be the device `stream` belongs to.  Its
 *   address is looked up once per device on the first call there (no
 *   allocation; hipGetSymbolAddress).  Every call on one GPU shares that
 *   GPU's array, so calls that overlap on one GPU (on different streams, or
 *   from different threads) race and must be serialised by the caller; calls
 *   on one stream are ordered and safe.  No part of it needs to start at
 *   zero (the statistics kernel writes every value it later reads).
 * Arguments and errors as tp_attn_shard_bwd without stats_i, plus TP_ENOSCRATCH.
 */
int tp_attn_shard_bwd_noalloc(const tp_attn_desc* desc, const void* dZ, const void* X, const void* Wqkv_i,
                              const void* Wo_i, const void* QKV_i, const void* O_i, const float* lse_i, void* dO_i,
                              void* dQKV_i, float* dWqkv_i, float* dWo_i, void* dX_i, void* stream);

/*
 * tp_sum_partials -- the all-reduce of operators g/f, emulated on one device
 * ([TP1] operators f and g; [L11] section 3 on the bias; [LP] I.III and [HJ] on dropout).
 *
 *   out = Dropout_{p, seed}( sum_{i=0}^{t-1} partials[i] + bias )
 * The sum runs in rank order in fp32; the bias is added exactly once after it.
 * Dropout keeps element (r, c) iff u >= floor(p * 2^32), where u is the high
 * 32 bits of output number (r*cols + c + 1) of a SplitMix64 stream seeded with
 * `seed` (Steele, Lea & Flood, OOPSLA 2014); kept elements are scaled by
 * 1/(1-p) in fp32.  The mask depends on neither t nor the tiling.
 * Arguments:
 *   rows, cols   tensor shape ([T, h] for the layer's all-reduces)
 *   t            number of partials, 1 <= t <= 64
 *   dtype        storage type of partials, bias and out
 *   partials     HOST array of t device pointers, each [rows, cols]
 *   bias         [cols] or NULL
 *   p_drop, seed dropout; p_drop = 0 disables it
 *   out          [rows, cols]; may alias none of the partials
 */
int tp_sum_partials(int64_t rows, int64_t cols, int32_t t, int32_t dtype, const void* const* partials,
                    const void* bias, float p_drop, uint64_t seed, void* out, void* stream);

/*
 * tp_sum_partials_residual -- the block-closing all-reduce with the residual
 * add fused ([LP] II.III Computational Details: fused bias + dropout +
 * residual add, fused all-reduce + residual add).
 *
 *   out = residual + Dropout_{p, seed}( sum_{i=0}^{t-1} partials[i] + bias )
 * As tp_sum_partials, with the residual (the block's input, [rows, cols],
 * same dtype, or NULL for none) added once, after dropout.  out may alias the
 * residual (in-place residual stream) but none of the partials.
 */
int tp_sum_partials_residual(int64_t rows, int64_t cols, int32_t t, int32_t dtype, const void* const* partials,
                             const void* bias, float p_drop, uint64_t seed, const void* residual, void* out,
                             void* stream);

/*
 * tp_reduce_scatter -- Megatron-SP's split of the block-closing all-reduce,
 * first half, emulated on one device ([LP] III.III Block Layout Contract).
 *
 * Rank `rank`'s token slice, rows [rank*rows/t, (rank+1)*rows/t), of
 *   residual + Dropout_{p, seed}( sum_i partials[i] + bias )
 * computed from those rows of the partials only.  The dropout mask of an
 * element is that of its position in the full [rows, cols] tensor, so the t
 * slices are exactly the rows of tp_sum_partials_residual's output.
 * Arguments:
 *   rows, cols   full tensor shape; rows % t != 0 gives TP_ENOTDIV
 *   rank         0 <= rank < t
 *   partials     HOST array of t device pointers, each the FULL [rows, cols] partial
 *   bias, p_drop, seed  as tp_sum_partials
 *   residual_r   [rows/t, cols] this rank's slice of the residual, or NULL
 *   out_r        [rows/t, cols] out
 */
int tp_reduce_scatter(int64_t rows, int64_t cols, int32_t t, int32_t rank, int32_t dtype,
                      const void* const* partials, const void* bias, float p_drop, uint64_t seed,
                      const void* residual_r, void* out_r, void* stream);

/* Token-wise norm of tp_sum_partials_norm and tp_reduce_scatter_norm. */
typedef enum {
  TP_NORM_RMS = 0,   /* y = x / sqrt(mean(x^2) + eps) * gamma */
  TP_NORM_LAYER = 1  /* y = (x - mean(x)) / sqrt(mean((x - mean(x))^2) + eps) * gamma + beta */
} tp_norm;

/*
 * tp_sum_partials_norm -- the block-closing all-reduce with the residual add
 * and the next sublayer's token-wise norm fused ([LP] II.III Computational
 * Details: fused layernorm / RMSnorm, fused bias + dropout + residual add).
 *
 *   out    = residual + Dropout_{p, seed}( sum_{i=0}^{t-1} partials[i] + bias )   (as tp_sum_partials_residual)
 *   normed = norm(out) over the cols features of each row
 * The norm reads out as stored (rounded to dtype); its statistics are fp32
 * sums in a fixed order, so every row's result is the same whichever call
 * computes it.
 * Arguments:
 *   rows, cols, t, dtype, partials, bias, p_drop, seed, residual  as tp_sum_partials_residual
 *   norm         TP_NORM_RMS or TP_NORM_LAYER
 *   gamma        [cols] gain (dtype), or NULL for ones
 *   beta         [cols] shift (dtype) for TP_NORM_LAYER, or NULL for zeros; must be NULL for TP_NORM_RMS
 *   eps          >= 0, finite
 *   out          [rows, cols] block output (the residual stream); may alias the residual
 *   normed       [rows, cols] its norm; may alias no other argument
 * Errors as tp_sum_partials_residual, plus TP_EINVAL for an unknown norm, a
 * bad eps, beta with TP_NORM_RMS or a NULL normed, and TP_EUNSUPPORTED for
 * rows of more than 32768 bf16 (16384 fp32) elements.
 */
int tp_sum_partials_norm(int64_t rows, int64_t cols, int32_t t, int32_t dtype, const void* const* partials,
                         const void* bias, float p_drop, uint64_t seed, const void* residual, int32_t norm,
                         const void* gamma, const void* beta, float eps, void* out, void* normed, void* stream);

/*
 * tp_reduce_scatter_norm -- Megatron-SP's reduce-scatter with the token-wise
 * norm on the rank's slice ([LP] III.III Block Layout Contract: after the
 * reduce-scatter each rank runs the layernorm / dropout of its own tokens;
 * [LP] II.III; [L11] section 3 places an RMSNorm before the Llama MLP).
 *
 * Rank `rank`'s token slice, rows [rank*rows/t, (rank+1)*rows/t), of
 * tp_sum_partials_norm's two outputs, computed from those rows of the
 * partials only; row for row bit-identical to tp_sum_partials_norm, so the
 * all-gather of the t normed slices is its normed output.
 * Arguments:
 *   rows, cols, t, rank, dtype, partials, bias, p_drop, seed, residual_r  as tp_reduce_scatter
 *   norm, gamma, beta, eps   as tp_sum_partials_norm
 *   out_r        [rows/t, cols] this rank's slice of the block output; may alias residual_r
 *   normed_r     [rows/t, cols] its norm (the slice the all-gather takes)
 * Errors as tp_reduce_scatter and tp_sum_partials_norm.
 */
int tp_reduce_scatter_norm(int64_t rows, int64_t cols, int32_t t, int32_t rank, int32_t dtype,
                           const void* const* partials, const void* bias, float p_drop, uint64_t seed,
                           const void* residual_r, int32_t norm, const void* gamma, const void* beta, float eps,
                           void* out_r, void* normed_r, void* stream);

/*
 * tp_all_gather -- Megatron-SP's second half, at the next block's entry,
 * emulated on one device ([LP] III.III Block Layout Contract).
 *
 *   out = [slices[0]; slices[1]; ...; slices[t-1]]   (rank order, exact copy)
 * Arguments:
 *   rows_per_rank, cols  shape of each slice; cols * element size must be a multiple of 16 bytes
 *   slices       HOST array of t device pointers, each [rows_per_rank, cols]
 *   out          [t * rows_per_rank, cols]; may alias none of the slices
 */
int tp_all_gather(int64_t rows_per_rank, int64_t cols, int32_t t, int32_t dtype, const void* const* slices,
                  void* out, void* stream);

/*
 * tp_comm_bytes -- host-only all-reduce accounting of one layer per microbatch
 * ([L11] section 5; [TP1] communication cost; [LP] II.II).  4 all-reduces
 * per layer (2 forward, 2 backward) of tokens*h*delta bytes each; a ring
 * all-reduce sends 2(t-1)/t of that per rank.  Touches no device.
 * Returns TP_EINVAL for tokens < 0, h < 0, t < 1, delta < 1 or out == NULL.
 */
int tp_comm_bytes(int64_t tokens, int64_t h, int32_t t, int32_t delta, tp_comm* out);

/*
 * tp_profile_arm -- profiling aid: time the library's next kernels with events.
 * `events` is a host array of n_events hipEvent_t handles (as void*), n_events
 * even and at most 64.  Each of the next n_events/2 step kernels the library
 * enqueues (one launch, or a launch and the small kernel finishing its split
 * part) takes one pair: events[2i] is stamped when its first dispatch starts
 * and events[2i+1] when its last one ends, by the dispatches themselves
 * (hipExtLaunchKernel), so no marker packet sits between kernels; after that
 * the hook is idle again.  n_events = 0 disarms it.  Process-wide: with
 * several threads launching, each step kernel claims the next free pair
 * under a lock, so which kernel gets which pair follows the order the
 * launches happen in.
 * Returns TP_EINVAL for an odd or out-of-range count or a NULL handle.
 */
int tp_profile_arm(void* const* events, int32_t n_events);

/*
 * tp_set_options -- process-wide launch options of every later call (host only).
 *   tile        TP_TILE_AUTO, or a tile shape every bf16 GEMM then takes
 *   split_tail  1 (default): a GEMM whose last round of tiles is at most half
 *               full splits it (over K into a caller buffer that the entry
 *               point documents as scratch, or over N in a paired launch),
 *               the attention kernels split their heaviest causal blocks, and
 *               the causal attention backward hands its dS tiles from dK/dV
 *               to dQ where they fit;
 *               0: no splits and no hand-over.
 * The results are the same either way up to fp32 rounding order (paired
 * half-width tails and dQ from handed-over tiles are bit-identical).  Returns TP_EINVAL for values outside
 * these ranges (the options are then unchanged).
 */
int tp_set_options(int32_t tile, int32_t split_tail);

/* tp_get_options -- the current options; TP_EINVAL for a NULL output. */
int tp_get_options(int32_t* tile, int32_t* split_tail);

/* Human-readable name of a status code (static string; never NULL). */
const char* tp_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* TP_SHARD_H */
