/*
 * tpshard.h -- C ABI of the MI355X (gfx950) tensor-parallel shard library.
 *
 * The library runs, on one GPU, the decode-time forward step of one
 * tensor-parallel (TP) shard of a Llama-style decoder block, and the dense
 * FFN block a chip holds under 2D weight-stationary partitioning:
 *
 *   attention stage  RMSNorm -> [int8 round trip] -> column-split QKV ->
 *                    RoPE + KV append -> grouped-query attention over the
 *                    shard's cache -> row-split W_O -> partial sum
 *                    -> [int8 block quantisation of the partial]
 *   merge            residual + sum of the shards' (dequantised) partials
 *   FFN stage        RMSNorm -> [int8 round trip] -> column-split W1/W3 +
 *                    SwiGLU -> row-split W2 -> partial -> [int8]
 *   merge            residual + sum of partials -> layer output
 *
 * and the final stage of the decode step, split over the vocabulary:
 *
 *   logits stage     final RMSNorm -> the shard's rows of the classifier
 *                    -> [int8 block quantisation of the logits slice]
 *   merge            the shards' (dequantised) slices placed side by side
 *
 * Sources: distributed-llama issue "[Feature Suggest] Tensor Parallellism for
 * Accelerating LLM" (buildLlama2Arch: the root/worker task list of one layer,
 * llamaRmsAttNorm .. llamaMergeFfn2, with quantise / sync / dequantise /
 * merge around the two partial-sum exchanges); aiterms.tw "Tensor
 * Parallelism" (核心概念: column and row split; 運作原理: the FFN walk-through
 * ending in an all-reduce of row-split partials); CS349E lecture 4
 * 03_pope_partitioning.py (demo 1: PaLM-540B FFN under 2D weight-stationary
 * partitioning; demo 3 observations: GQA head sharding without KV
 * replication while TP <= number of KV groups).
 *
 * Conventions shared by every entry point:
 *  - Every call returns an int32 status: TP_OK (0) or a negative TP_E* code.
 *    tp_last_error() gives a thread-local message for the last failure.
 *  - Device pointers are plain device addresses on the current HIP device;
 *    the library NEVER allocates or frees device memory. The caller sizes
 *    every device buffer from the byte counts init_shard returns.
 *  - Compute calls only enqueue work on the given hipStream_t (passed as
 *    void*; NULL = the null stream) and never synchronise. Argument errors
 *    are detected on the host before anything is enqueued.
 *  - Every device buffer must be 16-byte aligned (else TP_EALIGN).
 *  - A handle is not thread-safe; distinct handles are independent.
 *  - No C++ exception or abort crosses this boundary.
 */
#ifndef TPSHARD_H
#define TPSHARD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct tp_shard tp_shard; /* opaque host-side handle; owns no device memory */

enum { TP_F32 = 0, TP_BF16 = 1 };                         /* element types */
enum { TP_LLAMA_BLOCK = 0, TP_FFN_2D = 1, TP_LOGITS = 2, TP_ATTN_BATCH = 3 }; /* tp_config.kind */
enum { TP_A2A_HEADS_TO_BATCH = 0, TP_A2A_BATCH_TO_HEADS = 1 };       /* tp_all_to_all direction */
enum { TP_STAGE_ATTN = 0, TP_STAGE_FFN = 1, TP_STAGE_LOGITS = 2 };   /* decode_step / merge_partials stage */
/* tp_config.quant bit mask. TP_Q_PARTIALS / TP_Q_INPUTS: the block-32 int8
 * round trip of the exchanged partials / the normalised stage inputs
 * (distributed-llama issue, buildLlama2Arch: the quantise / sync / dequantise
 * tasks). TP_Q_WEIGHTS: weight-only int8 projections (CS349E lecture 4,
 * 03_pope_partitioning.py, demo 4: small-batch decode is bound by the weight
 * bytes, and int8 weights cut the measured PaLM decode time): load_weights
 * cuts every row of Wq/Wk/Wv/Wo/W1/W3/W2 (the shard's slice, given in
 * w_dtype) into blocks of 32 along k and stores each block with the same
 * codec as an fp32 scale and 32 int8 codes; the projections then accumulate
 * sum_blocks scale * sum_k code * x in fp32. Needs dim, Hq/T*head_dim and F/T
 * multiples of 32. Not for TP_FFN_2D. */
enum { TP_Q_NONE = 0, TP_Q_PARTIALS = 1, TP_Q_INPUTS = 2, TP_Q_WEIGHTS = 4 };

enum {
    TP_OK = 0,
    TP_EINVAL = -1,   /* bad configuration, enum, size or null pointer */
    TP_EALIGN = -2,   /* a device pointer is not 16-byte aligned */
    TP_ESTATE = -3,   /* call out of order (e.g. decode_step before load_weights) */
    TP_ENODEV = -4,   /* no HIP device, or the current device is not gfx950 */
    TP_EHIP = -5,     /* a HIP runtime call or kernel launch failed */
    TP_ENOTIMPL = -6  /* valid request the library does not implement */
};

/* Bits of the device error word (first 4 bytes of the workspace). */
enum {
    TP_DERR_LEN = 1,    /* some lens[b] was < 0 or >= max_ctx; that sequence was skipped */
    TP_DERR_HANDOFF = 2 /* in the one-launch QKV projection + attention (decode_step, batch
                           <= 4), an attention workgroup waited 0.17 s for its queries and
                           went on without them: that stage's outputs are invalid */
};

/*
 * Shard configuration. Sizes are those of the FULL (unsharded) model; the
 * library derives the shard's slice from tp_size / tp_rank:
 *   q heads  [r*Hq/T, (r+1)*Hq/T), kv heads [r*Hkv/T, (r+1)*Hkv/T),
 *   FFN features [r*F/T, (r+1)*F/T)  (column split of Wq/Wk/Wv/W1/W3,
 *   row split of Wo/W2: the shard multiplies its column slice of Wo/W2).
 * q head h uses kv head h / (Hq/Hkv) (contiguous groups).
 *
 * kind == TP_LLAMA_BLOCK: w_dtype TP_F32 or TP_BF16, kv_dtype likewise;
 *   requires Hq % Hkv == 0, Hq % T == 0, Hkv % T == 0, F % T == 0,
 *   hd in {16, 32, 48, 64, 128}, at most 8 q heads per kv head,
 *   max_batch <= 16, dim, Hq_s*hd and F/T multiples of 8 (bf16) or 4 (fp32)
 *   elements, dim % 32 == 0 when quant != 0, quant_block == 32, and the
 *   attention workgroup's LDS (which grows with max_ctx) within 64 KiB.
 * kind == TP_FFN_2D: dim = E (the block's E slice), ffn_hidden = F (the
 *   block's F slice), w_dtype TP_BF16, tp_size 1, heads ignored, quant 0;
 *   E a multiple of 576, 2F of 288 and F of 64; any max_batch >= 1. The
 *   decode step is Y = (silu(X W_gate^T) * (X W_in^T)) W_out^T.
 * kind == TP_LOGITS: the final stage (distributed-llama issue,
 *   buildLlama2Arch: llamaRmsFinal, llamaRmsFinalNorm, llamaLogits,
 *   llamaQuantizeLogits, llamaSyncLogits, llamaDequantizeLogits,
 *   llamaMergeLogits). dim = D, ffn_hidden = V (the vocabulary); the shard
 *   owns the logits [r*V/T, (r+1)*V/T) (column split of the classifier over
 *   the vocabulary); w_dtype TP_F32 or TP_BF16; heads, head_dim, max_ctx
 *   and kv_dtype ignored; quant may hold TP_Q_PARTIALS (int8 wire of the
 *   logits slice) and TP_Q_WEIGHTS (int8 classifier), not TP_Q_INPUTS (the
 *   page lists no quantisation of the final norm's output); requires V % T
 *   == 0, max_batch <= 16, D a multiple of 8 (32 with int8 weights), V/T a
 *   multiple of 8 (32 with TP_Q_PARTIALS).
 * kind == TP_ATTN_BATCH: batch-sharded attention (CS349E lecture 4,
 *   03_pope_partitioning.py, demo 3 observations: with fewer KV heads than
 *   shards, head sharding would keep a KV head on several shards; sharding
 *   by sequence keeps each sequence's KV once, with every head local, and
 *   the queries and outputs cross an all-to-all). max_batch = B, the batch of
 *   the whole layer; shard r owns sequences [r*B/T, (r+1)*B/T) with all
 *   n_heads q and n_kv_heads kv heads; n_heads, n_kv_heads, head_dim,
 *   max_ctx, kv_dtype and rope_theta as for TP_LLAMA_BLOCK; dim, ffn_hidden,
 *   w_dtype and norm_eps ignored; quant 0. Requires B % T == 0, Hq % Hkv
 *   == 0, Hq % T == 0 (the head shards on the other side of the all-to-all),
 *   the head_dim, q-heads-per-kv-head and LDS rules of TP_LLAMA_BLOCK, and
 *   B <= 16 * T.
 */
typedef struct {
    int32_t kind;
    int32_t dim, n_heads, n_kv_heads, head_dim, ffn_hidden;
    int32_t tp_size, tp_rank;
    int32_t max_batch, max_ctx; /* max_ctx = KV positions per sequence (cached + new) */
    int32_t w_dtype, kv_dtype;
    int32_t quant, quant_block;
    float rope_theta; /* default 10000 */
    float norm_eps;   /* default 1e-5 */
} tp_config;

/* Byte counts of the caller-owned device buffers. */
typedef struct {
    uint64_t packed_weights; /* the shard's packed weights, gains and RoPE table */
    uint64_t kv_cache_each;  /* one of K or V: [max_batch][Hkv_s][max_ctx][hd] kv_dtype */
    uint64_t workspace;      /* activations between kernels, the device error word and (batch
                                <= 4 one-launch QKV + attention) a step counter: one workspace
                                per handle, kept between calls */
    uint64_t wire;           /* one shard's exchanged partial for max_batch rows */
} tp_sizes;

/* FULL layer weights on the device, (out, in) row-major, element type
 * w_dtype: wq [Hq*hd][D], wk/wv [Hkv*hd][D], wo [D][Hq*hd], w1/w3 [F][D],
 * w2 [D][F]; g_att/g_ffn fp32 [D] RMSNorm gains.
 * For TP_FFN_2D: w1 = W_gate [F][E], w3 = W_in [F][E], w2 = W_out [E][F]
 * (bf16); the others are ignored and may be NULL.
 * For TP_LOGITS: w1 = W_cls [V][D] (w_dtype), g_att = fp32 [D] final RMSNorm
 * gain; the others are ignored and may be NULL. */
typedef struct {
    const void *wq, *wk, *wv, *wo, *w1, *w3, *w2;
    const float *g_att, *g_ffn;
} tp_layer_weights;

/* Optional fp32 device outputs of intermediate values (NULL = not written);
 * rows are the batch:
 *  xn   [B][D]          normalised stage input (after the int8 round trip if any)
 *  q    [B][Hq_s*hd]    rotated queries            (attention stage)
 *  k, v [B][Hkv_s*hd]   rotated keys, values        (attention stage)
 *  att  [B][Hq_s*hd]    attention outputs           (attention stage)
 *  a    [B][F_s]        SwiGLU activations          (FFN stage)
 *  p_pre [B][D]         the stage's fp32 partial before quantisation
 *  xq   [B][D]          normalised stage input BEFORE the int8 round trip
 *                       (the fp32 row the quantiser of TP_Q_INPUTS codes;
 *                       equal to xn when that bit is off) */
typedef struct {
    float *xn, *q, *k, *v, *att, *a, *p_pre, *xq;
} tp_taps;

/*
 * init_shard: validate cfg, plan the shard's slice and return a host handle
 * and the device buffer sizes. The slice follows aiterms.tw "Tensor
 * Parallelism", 核心概念 items 1 and 2: the shard keeps whole output rows of
 * the column-split projections (its q / kv heads of Wq, Wk, Wv and its FFN
 * features of W1, W3) and the matching input columns of the row-split ones
 * (Wo, W2), whose products are full-size partials to be summed. Host only: enqueues nothing and needs no GPU.
 * Errors: TP_EINVAL (null pointer, unknown enum, shape rule above broken).
 */
int32_t init_shard(const tp_config *cfg, tp_shard **out, tp_sizes *sizes);

/*
 * load_weights: slice the shard's part out of the FULL layer weights and
 * pack it into `packed` (layout private to the library; the slices are those
 * of aiterms.tw "Tensor Parallelism", 核心概念 items 1-2, and the KV heads a
 * shard owns follow CS349E lecture 4, 03_pope_partitioning.py, demo 3
 * observations: with TP up to the number of KV heads, each KV head lives on
 * exactly one shard), compute the RoPE
 * cos/sin table (fp64 on the device, stored fp32) into `packed`, clear the
 * device error word in `workspace`, and remember k_cache / v_cache /
 * workspace for later calls. Enqueued on hip_stream; the caller must keep
 * `full` alive until the stream reaches this point.
 * k_cache / v_cache hold [max_batch][Hkv_s][max_ctx][hd] kv_dtype each (the
 * caller fills the cached past positions; the library appends); they are
 * unused (may be NULL) for TP_FFN_2D and TP_LOGITS. For TP_ATTN_BATCH no
 * weight is read (all of `full`'s pointers may be NULL) and the caches hold
 * [B/T][Hkv][max_ctx][hd] kv_dtype each.
 * Errors: TP_EINVAL, TP_EALIGN, TP_ENODEV, TP_EHIP.
 */
int32_t load_weights(tp_shard *s, const tp_layer_weights *full, void *packed, void *k_cache,
                     void *v_cache, void *workspace, void *hip_stream);

/*
 * decode_step: one stage of the shard's decode step for `batch` rows: the
 * worker side of one layer of distributed-llama issue "[Feature Suggest]
 * Tensor Parallellism for Accelerating LLM", buildLlama2Arch (attention
 * stage: llamaRmsAttNorm, llamaQuantizeRmsAtt, llamaQkv, llamaMultiheadAtt,
 * llamaAttOutput, llamaQuantizeAtt; FFN stage: llamaRmfFfnNorm,
 * llamaQuantizeRmfFfn, llamaFfn, llamaFfn2, llamaQuantizeFfn2), with every
 * shard normalising its own input instead of receiving the root's.
 *  stage TP_STAGE_ATTN: x = fp32 [batch][D] residual input; lens = device
 *    int32 [batch] cached positions per sequence: the new token's K/V are
 *    written at slot lens[b] and attention covers lens[b] + 1 positions.
 *    The library never advances lens. A sequence with lens[b] outside
 *    [0, max_ctx) is skipped (attention output 0) and TP_DERR_LEN is set in
 *    the device error word.
 *  stage TP_STAGE_FFN: x = fp32 [batch][D] (the merged attention output);
 *    lens unused (may be NULL).
 *  For TP_FFN_2D only TP_STAGE_FFN is valid: x = bf16 [batch][E], and
 *    wire_out receives Y fp32 [batch][E] (batch <= max_batch, any size).
 *  For TP_LOGITS only TP_STAGE_LOGITS is valid: x = fp32 [batch][D] (the
 *    last layer's merged output); wire_out receives the shard's logits
 *    [batch][V/T] in the wire format below (row length V/T instead of D);
 *    the taps xn (final-normalised rows) and p_pre (fp32 logits slice) are
 *    written, the others ignored.
 *  For TP_ATTN_BATCH only TP_STAGE_ATTN is valid: x = fp32
 *    [batch][(Hq + 2*Hkv)*hd] rows of the shard's sequences (batch <= B/T):
 *    the raw (unrotated) q of every q head, then k and v of every kv head
 *    (what the all-to-all of the queries and the shard's own K/V projection
 *    deliver); lens = device int32 [batch] as for the attention stage above
 *    (slot lens[b] of cache row b); wire_out receives the attention outputs
 *    fp32 [batch][Hq*hd]; the taps q, k, v (rotated) and att are written.
 *  wire_out: the partial this shard exchanges. With TP_Q_PARTIALS: int8
 *    codes [batch][D] at offset 0, then fp32 scales [batch][D/32] at the
 *    offset tp_wire_scales_offset(cfg, batch) (one scale per 32 consecutive
 *    elements of a row: scale = max|p| / 127, code = p / scale rounded half
 *    away from zero, clamped to +-127; an all-zero block has scale 0).
 *    Otherwise fp32 [batch][D].
 *  taps: NULL or optional intermediate outputs (tp_taps).
 *  At batch <= 4 with a bf16 cache of head dim 128 and at most 2 q heads per
 *  kv head, the attention stage runs the QKV projection, the chunk
 *  attention and the combine of the chunks as one launch (queries and chunk
 *  records handed between its workgroups as tagged words); the results are
 *  bitwise those of the separate launches.
 * Errors: TP_EINVAL, TP_EALIGN, TP_ESTATE (no load_weights yet), TP_EHIP.
 */
int32_t decode_step(tp_shard *s, int32_t stage, const void *x, const int32_t *lens,
                    int32_t batch, void *wire_out, const tp_taps *taps, void *hip_stream);

/*
 * decode_step_noalloc: decode_step for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). Same kernels, arguments and results as decode_step
 * (the QKV projection and the attention always as separate launches), but
 * the per-step buffers (the workspace's regions) live in one static device
 * array of the library, 16 MiB per GPU, held until the process ends; the
 * handle's workspace, if any, is not used, and a TP_LLAMA_BLOCK handle may be
 * loaded with workspace = NULL (its other stage calls then return
 * TP_ESTATE). The array's address on each device is looked up when a handle
 * is loaded on it. Nothing is allocated, freed or created by this call.
 *  err_out: NULL or a device uint32 (4-byte aligned) into which the TP_DERR_*
 *    bits of this call are ORed (the library never clears it).
 *  Every call on one GPU uses that GPU's array: calls that overlap on one GPU
 *  (concurrent streams, or host threads) race and must be serialised by the
 *  caller. Each call writes every buffer region before reading it, so no state
 *  carries over between calls.
 *  The kernel-timing probe is not used by this call.
 * Errors: those of decode_step; TP_EINVAL for a kind other than
 * TP_LLAMA_BLOCK or a shard whose workspace (tp_sizes.workspace) exceeds the
 * 16 MiB array; TP_EALIGN for a misaligned err_out.
 */
int32_t decode_step_noalloc(tp_shard *s, int32_t stage, const void *x, const int32_t *lens,
                            int32_t batch, void *wire_out, const tp_taps *taps, uint32_t *err_out,
                            void *hip_stream);

/*
 * merge_partials (distributed-llama issue, buildLlama2Arch: llamaSyncAtt /
 * llamaDequantizeAtt / llamaMergeAtt and their FFN counterparts; aiterms.tw
 * "Tensor Parallelism", 運作原理: the row-split partials' all-reduce):
 * out = residual + sum_{i < n_wires} dequant(wires[i]) in the
 * order of the array (shard order), per element, in fp32; `wires` is a HOST
 * array of n_wires device pointers in this shard's wire format. out may
 * alias residual. fp32 [batch][D] throughout.
 * Errors: TP_EINVAL (n_wires < 1 or > 64, null pointers), TP_EALIGN, TP_EHIP.
 */
int32_t merge_partials(const tp_shard *s, int32_t stage, const void *const *wires,
                       int32_t n_wires, const float *residual, float *out, int32_t batch,
                       void *hip_stream);

/*
 * decode_merge_step: decode_step, then merge_partials of this stage's
 * partials onto x, with the merge done by the kernel that writes this shard's
 * own partial (the down-projection's store, or the int8 quantiser) instead of
 * a kernel of its own: the row-split partials' all-reduce fused into their
 * producer (same passages as decode_step and merge_partials).
 *  x_out = x + sum_{i < n_wires} dequant(wires[i]) in array order, bitwise
 *    what merge_partials(wires, n_wires, residual = x) writes. Exactly one
 *    wires[i] must equal wire_out: that term is this shard's partial, taken
 *    from the producing kernel's registers; the others are read from memory
 *    and must be complete when the call is enqueued (earlier work on the
 *    stream). TP_LLAMA_BLOCK only.
 *  x_out may alias x, but not a wire (TP_EINVAL).
 *  Other arguments as in decode_step and merge_partials.
 * Errors: those of decode_step and merge_partials; TP_EINVAL when wire_out is
 * not in wires, appears twice, or x_out equals a wire.
 */
int32_t decode_merge_step(tp_shard *s, int32_t stage, const void *x, const int32_t *lens,
                          int32_t batch, void *wire_out, const void *const *wires,
                          int32_t n_wires, float *x_out, const tp_taps *taps, void *hip_stream);

/*
 * merge_logits: the full logits rows from every shard's logits wire
 * (distributed-llama issue, buildLlama2Arch: llamaSyncLogits,
 * llamaDequantizeLogits, llamaMergeLogits): out fp32 [batch][V], columns
 * [i*V/T, (i+1)*V/T) = dequant(wires[i]) ((float)code * scale per element,
 * or the fp32 values as they are). `wires` is a HOST array of n_wires = T
 * device pointers in shard order, each a wire decode_step wrote for `batch`
 * rows with a TP_LOGITS handle of the same configuration. out must not
 * overlap a wire. TP_LOGITS only.
 * Errors: TP_EINVAL (wrong kind, n_wires != T, null pointers, out equal to a
 * wire), TP_EALIGN, TP_EHIP.
 */
int32_t merge_logits(const tp_shard *s, const void *const *wires, int32_t n_wires, float *out,
                     int32_t batch, void *hip_stream);

/*
 * tp_all_to_all: the two re-shardings around batch-sharded attention, seen
 * from shard r of a TP_ATTN_BATCH handle (same passage as TP_ATTN_BATCH),
 * for the whole batch B = max_batch, with nb = B/T and C = (Hq/T)*hd:
 *  TP_A2A_HEADS_TO_BATCH: srcs[i] = head shard i's rows [B] (row stride
 *    ld_src >= C elements; its q heads [i*Hq/T, (i+1)*Hq/T) in columns
 *    [0, C)) -> dst [nb] rows (stride ld_dst >= T*C): row b gets sequence
 *    r*nb + b of every head, head shard i's columns at [i*C, (i+1)*C).
 *  TP_A2A_BATCH_TO_HEADS: srcs[i] = batch shard i's rows [nb] (stride
 *    ld_src >= T*C; every head) -> dst [B] rows (stride ld_dst >= C): row b
 *    gets columns [r*C, (r+1)*C) of row b % nb of srcs[b / nb].
 *  Every value is copied unchanged. `srcs` is a HOST array of n_srcs = T
 *  device pointers; ld_src and ld_dst are multiples of 4, buffers 16-byte
 *  aligned; dst must not overlap a source. Other columns of dst are left as
 *  they are (so the queries can land in the first columns of the attention
 *  input rows).
 * Errors: TP_EINVAL (wrong kind or direction, n_srcs != T, strides too
 * small or not multiples of 4, null pointers), TP_EALIGN, TP_EHIP.
 */
int32_t tp_all_to_all(const tp_shard *s, int32_t dir, const void *const *srcs, int32_t n_srcs,
                      int64_t ld_src, float *dst, int64_t ld_dst, void *hip_stream);

/* Byte offset of the fp32 scales inside a quantised wire of `batch` rows
 * (16-byte aligned, right after the int8 codes; rows of D elements, of V/T
 * for TP_LOGITS). */
uint64_t tp_wire_scales_offset(const tp_config *cfg, int32_t batch);

/* TP_Q_WEIGHTS: where projection `proj` (0 = Wqkv, 1 = Wo, 2 = W13 with the
 * W1_f / W3_f rows interleaved, 3 = W2) sits inside the packed weights: its
 * int8 codes [rows][cols] at byte *codes_off, its fp32 scales
 * [rows][cols / 32] at byte *scales_off, both row-major (scale j of a row
 * covers codes 32 j .. 32 j + 31). For TP_LOGITS, proj 0 is the shard's
 * classifier rows [V/T][D]. TP_EINVAL for a handle without int8 weights, an
 * unknown proj or a null output. */
int32_t tp_packed_int8_view(const tp_shard *s, int32_t proj, uint64_t *codes_off,
                            uint64_t *scales_off, int32_t *rows, int32_t *cols);

/* Reads (and clears, when clear != 0) the device error word in the handle's
 * workspace; synchronises hip_stream. */
int32_t tp_read_error_word(tp_shard *s, uint32_t *word, int32_t clear, void *hip_stream);

/*
 * Kernel timing probe: while armed, the library records a HIP event pair
 * (created with hipEventDisableSystemFence, so the pair adds well under a
 * microsecond to what it brackets) on the launch stream around every launch
 * of kernel `kernel_id` (see tp_kernel_name) it enqueues, and accumulates the
 * elapsed time of completed pairs. tp_kernel_timing_arm(s, -1) disarms. Reading synchronises
 * on the recorded events. Host-side HIP events only; no device memory.
 */
int32_t tp_kernel_timing_arm(tp_shard *s, int32_t kernel_id);
int32_t tp_kernel_timing_read(tp_shard *s, double *total_ms, int32_t *launches);
const char *tp_kernel_name(int32_t kernel_id); /* NULL past the last id */

/*
 * tp_handoff_test: for tests of the error path of the one-launch QKV +
 * attention (decode_step, batch <= 4, see TP_DERR_HANDOFF). Sets, for the
 * handle's later attention stages, the longest wait for another workgroup's
 * values in ticks of the 100 MHz real-time counter (0: the normal 2^24) and a
 * mask XORed into the tag the waiting workgroups look for (nonzero: a tag no
 * word carries, so every wait runs out and TP_DERR_HANDOFF is set; the
 * stage's outputs are then invalid). tp_handoff_test(s, 0, 0) restores the
 * normal behaviour. Host only; errors: TP_EINVAL (null handle).
 */
int32_t tp_handoff_test(tp_shard *s, uint32_t wait_ticks, uint32_t tag_xor);

/*
 * Measured-peak probes: the benchmark's measured denominators, not steps of
 * the shard. Enqueue only; the caller times them (HIP events).
 *  tp_probe_read: `blocks` workgroups read [buf, buf + bytes) once, each a
 *    contiguous span, with 16-byte nontemporal loads, eight per thread in
 *    flight; out receives one uint32 per workgroup (an XOR of what it read).
 *  tp_probe_mfma: `blocks` workgroups of 4 waves each run iters x 4
 *    independent bf16 MFMAs (32 x 32 x 16: 32768 flops each) per wave from
 *    registers, no memory traffic; out receives blocks * 256 floats.
 *  Buffers 16-byte aligned; 1 <= blocks <= 2^20, iters >= 1.
 * Errors: TP_EINVAL, TP_EALIGN, TP_ENODEV, TP_EHIP.
 */
int32_t tp_probe_read(const void *buf, uint64_t bytes, uint32_t *out, int32_t blocks, void *hip_stream);
int32_t tp_probe_mfma(int32_t blocks, int32_t iters, float *out, void *hip_stream);

void destroy_shard(tp_shard *s);
const char *tp_status_str(int32_t status);
const char *tp_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TPSHARD_H */
