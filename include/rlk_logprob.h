/*
 * rlk_logprob.h — C ABI of the strict-path selected-token logprob on MI355X (gfx950).
 *
 * The library computes, for every row t of a hidden-state matrix h[T,H] and its target token y_t,
 *
 *     z[t,v]  = sum_k h[t,k] * W[v,k]                      (the LM-head projection, W is [V,H])
 *     z'      = z * inv_temperature
 *     lse[t]  = log sum_v exp(z'[t,v])
 *     logp[t] = z'[t,y_t] - lse[t]
 *     entropy[t] = lse[t] - sum_v softmax(z')[t,v] * z'[t,v]          (optional)
 *
 * under one fixed numeric contract, so that each row's outputs are bitwise identical however the
 * rows are laid out: one packed training batch, ragged rollout batches, row chunks of any size,
 * or the vocabulary split into contiguous shards whose partial results are merged.
 *
 * Sources (pages about RL-Kernel, vime and vLLM on ROCm):
 *  - RL-Kernel v0.1.0 summary (agentlenshq.com), section "Numeric execution contract": a forward
 *    fixes its inputs, how a reduction is split, the merge order of partial results, precisions,
 *    rounding points and math primitives. Same page, strict-path boundary table, row "Linear
 *    logprob": actual vocab range, target ownership, local reduction, cross-rank LSE merge. Same
 *    page, ROCm fixes list: deterministic MFMA GEMM; vocab reduction and the cross-TP vocab merge.
 *  - nxbn.cn blog on bitwise train/rollout consistency, §3.1 (the logprob is log_softmax at the
 *    token; its max and sum reductions decide the last bits), §3.2 (a fixed reduction tree with
 *    fp32 intermediates; wave64 shuffle steps in a fixed order), §3.3 (the rollout recomputes the
 *    logprob from hidden states and tokens), §3.4 (no FMA contraction; 256-byte alignment).
 *  - kongchang.com article on bit-for-bit logprob alignment, "four key links": reduction order,
 *    intermediate precision, rounding points, math primitives.
 * The numeric contract itself (tile width, merge trees, primitives) is spelled out at
 * rlk_logprob_contract_id() and in the library's kernel source.
 *
 * Conventions for every entry point:
 *  - Device pointers are HIP device memory owned by the caller; the library never frees them.
 *    Host pointers are marked "host". Every device pointer must be 16-byte aligned; a misaligned
 *    pointer returns RLK_ERR_ALIGNMENT (there is no second code path for it).
 *  - Matrices are row-major with unit stride along the hidden dimension (row stride = H).
 *    hidden and W are bfloat16 bit patterns (2 bytes each); rms_gamma is bfloat16 [H].
 *  - targets are int32 [T]; a negative target marks a padded row: its logp, lse and entropy are
 *    written as +0.0. A target >= V writes NaN for that row and sets RLK_DEVICE_STATUS_BAD_TARGET
 *    in the workspace status word (see rlk_logprob_device_status).
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream of the handle's device)
 *    and runs asynchronously; forward, partials and merge neither allocate nor synchronize.
 *  - No exception crosses the ABI. On failure nothing is enqueued, the status says why, and
 *    rlk_last_error() holds a message (thread-local, valid until the next call on the thread).
 *  - A handle is immutable after creation and may be used from several threads; calls that
 *    share a workspace must be ordered by the caller (same stream or events).
 */
#ifndef RLK_LOGPROB_H
#define RLK_LOGPROB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct rlk_logprob* rlk_logprob_t;
typedef void* rlk_stream_t; /* hipStream_t */

typedef enum rlk_status {
  RLK_OK = 0,
  RLK_ERR_INVALID_ARGUMENT = 1, /* null pointer, negative size, inconsistent layout */
  RLK_ERR_NO_DEVICE = 2,        /* no HIP device, or the device index does not exist */
  RLK_ERR_UNSUPPORTED_ARCH = 3, /* device is not gfx950 */
  RLK_ERR_UNSUPPORTED_SHAPE = 4,/* H not a multiple of 128, V not a multiple of the segments ... */
  RLK_ERR_ALIGNMENT = 5,        /* a device pointer is not 16-byte aligned */
  RLK_ERR_WORKSPACE = 6,        /* workspace missing or smaller than the size query returned */
  RLK_ERR_CONTRACT = 7,         /* shard range not on segment boundaries, flags mismatch */
  RLK_ERR_HIP = 8               /* a HIP runtime call failed (message in rlk_last_error) */
} rlk_status_t;
/* Deliberate limits of this build:
 *  - H must be a multiple of 128 (not merely of the MFMA's 32): every kernel stages K in steps of
 *    64 and peels its last two steps, which keeps the K loops free of remainder code. Other H
 *    are refused with RLK_ERR_UNSUPPORTED_SHAPE, never run a second way.
 *  - There is no separate "build failed" status: the library is a prebuilt gfx950 code object,
 *    so a missing or foreign build fails to load (the binding refuses to run without it), and a
 *    device that is not gfx950 gets RLK_ERR_UNSUPPORTED_ARCH at rlk_logprob_create. */

/* rlk_logprob_config_t.flags */
#define RLK_FLAG_RMSNORM 1u /* apply the final RMSNorm (rms_gamma, rms_eps) to hidden first */
#define RLK_FLAG_ENTROPY 2u /* also produce the per-row entropy of softmax(z') */
/* Software EXP, LOG and RSQ built only from IEEE fp32 operations rounded to nearest even (the
 * "primitives" item of the numeric execution contract on the RL-Kernel v0.1.0 summary page asks
 * that they be fixed; this fixes them independently of the GPU's transcendental units). With it
 * every output bit follows from the inputs through operations any IEEE-754 machine performs
 * identically, so a CPU model of the contract reproduces logp, lse and entropy bit for bit
 * whenever it reproduces the logits. Costs extra VALU work in the tile epilogue. Part of the
 * contract id: results differ from the default mode (both stay within 1e-3 of exact). */
#define RLK_FLAG_PORTABLE_EXP 4u

/* bits of the device status word */
#define RLK_DEVICE_STATUS_BAD_TARGET 1u

/* Numeric configuration, fixed at creation. Every field is part of the contract id. */
typedef struct rlk_logprob_config {
  int32_t hidden_size;     /* H: a multiple of 128, at most 65536 */
  int32_t vocab_segments;  /* S_c: 1, 2, 4 or 8 contiguous vocab segments (contract split) */
  int64_t vocab_size;      /* V: a multiple of S_c; V / S_c at most 2^24 */
  float inv_temperature;   /* fl32(1/tau) multiplied into every logit; 1.0f = no temperature */
  float rms_eps;           /* epsilon inside the RMSNorm square root (RLK_FLAG_RMSNORM) */
  uint32_t flags;          /* RLK_FLAG_* */
  uint32_t reserved;       /* must be 0 */
} rlk_logprob_config_t;

/* How the rows and the vocabulary are presented to one forward call. None of it changes a
 * row's arithmetic; it only changes launches, so outputs are bitwise identical for any layout. */
typedef struct rlk_layout_desc {
  int64_t num_rows;             /* T >= 0 */
  int32_t num_batches;          /* 0 or 1: one packed batch (training layout); >1: ragged batches */
  int32_t vocab_shards;         /* 1..S_c, dividing S_c: W processed as that many row ranges */
  const int64_t* batch_offsets; /* host [num_batches+1], ascending, [0] = 0, [nb] = T; or NULL */
  int64_t row_chunk;            /* >0: each batch runs in launches of at most this many rows */
  int32_t token_tile;           /* 0 = chosen per launch; or 32, 64, 128, 256 rows per block */
  int32_t reserved;             /* must be 0 */
} rlk_layout_desc_t;

/* Per-row, per-vocab-segment partial record, as exchanged between vocab shards.
 * m = max_v z' over the segment, s = sum_v exp(z' - m), u = sum_v exp(z' - m) (z' - m)
 * (0 without RLK_FLAG_ENTROPY), tgt = z'[t, y_t] when the segment owns y_t, else NaN. */
typedef struct rlk_segment_record {
  float m, s, u, tgt;
} rlk_segment_record_t;

/* Create a handle bound to HIP device `device`. Checks the device exists and is gfx950 and that
 * the configuration is supported. Returns RLK_ERR_NO_DEVICE on a machine without a GPU. */
rlk_status_t rlk_logprob_create(const rlk_logprob_config_t* config, int device,
                                rlk_logprob_t* out);

/* Destroy a handle (host state only). NULL is accepted. */
rlk_status_t rlk_logprob_destroy(rlk_logprob_t handle);

/* Host-only, no device needed: bytes of device workspace rlk_logprob_forward needs for this
 * configuration and layout. */
rlk_status_t rlk_logprob_workspace_size(const rlk_logprob_config_t* config,
                                        const rlk_layout_desc_t* layout, size_t* bytes);

/* Host-only, no device needed: validates a layout against a configuration and reports how many
 * LM-head kernel launches a forward with it makes (row launch groups x vocab shards). */
rlk_status_t rlk_layout_check(const rlk_logprob_config_t* config,
                              const rlk_layout_desc_t* layout, int64_t* num_launches);

/* The strict-path forward: the LM-head projection, log-softmax over the vocabulary and the
 * target token's logprob (nxbn.cn blog §3.1; the "Linear logprob" row of the strict-path
 * boundary table on the RL-Kernel v0.1.0 summary page), recomputed from hidden states and tokens
 * (nxbn.cn blog §3.3), optionally after the final RMSNorm (the same table's "RMSNorm" row).
 * hidden: bf16 [T,H]; W_lm: bf16 [V,H]; targets: int32 [T];
 * rms_gamma: bf16 [H] with RLK_FLAG_RMSNORM, else NULL. Outputs fp32 [T]: logp, lse, and
 * entropy (required with RLK_FLAG_ENTROPY, else NULL). workspace: device memory of at least
 * rlk_logprob_workspace_size bytes, 256-byte aligned; its contents on entry do not matter. */
rlk_status_t rlk_logprob_forward(rlk_logprob_t handle, const void* hidden, const void* W_lm,
                                 const int32_t* targets, const rlk_layout_desc_t* layout,
                                 const void* rms_gamma, float* logp, float* lse, float* entropy,
                                 void* workspace, size_t workspace_bytes, rlk_stream_t stream);

/* rlk_logprob_forward that also records caller-created HIP events (hipEvent_t) on `stream`:
 * events[2i] right before and events[2i+1] right after the i-th LM-head kernel launch, for
 * i < num_events / 2 (extra launches are not bracketed). For measuring that kernel's duration
 * with the caller's clock; the results are bit-identical to rlk_logprob_forward. */
rlk_status_t rlk_logprob_forward_timed(rlk_logprob_t handle, const void* hidden, const void* W_lm,
                                       const int32_t* targets, const rlk_layout_desc_t* layout,
                                       const void* rms_gamma, float* logp, float* lse,
                                       float* entropy, void* workspace, size_t workspace_bytes,
                                       rlk_stream_t stream, void* const* events,
                                       int32_t num_events);

/* ---- Allocation-free forward ----------------------------------------------------------------
 * For callers that cannot allocate device memory: code being captured into a HIP graph, tight
 * serving loops, harnesses that forbid hipMalloc. rlk_logprob_forward with the same arguments
 * and results (bit for bit), except that the workspace is a fixed array in device memory that
 * the library holds, one per GPU, RLK_NOALLOC_SCRATCH_BYTES (64 MiB) large, present from library
 * load until the process ends. Nothing is allocated: no hipMalloc, hipFree or allocating library
 * call; the caller still passes inputs and outputs.
 *  - A layout whose rlk_logprob_workspace_size exceeds RLK_NOALLOC_SCRATCH_BYTES is refused with
 *    RLK_ERR_WORKSPACE before anything is enqueued (about 19 KB per row at V = 151936 with four
 *    segments, 28.5 KB with entropy: some 3400 / 2300 rows per call).
 *  - Every call on one GPU uses that GPU's one array, and the array keeps the last call's
 *    contents (the forward clears what must start at zero itself). Calls that overlap in time on
 *    one GPU race: order them (one stream, or events) even across handles.
 *  - The device status word of these calls lives in that array, not in a caller workspace, so
 *    rlk_logprob_device_status cannot read it; a target >= V still writes NaN for its row. */
#define RLK_NOALLOC_SCRATCH_BYTES (64u << 20)
rlk_status_t rlk_logprob_forward_noalloc(rlk_logprob_t handle, const void* hidden,
                                         const void* W_lm, const int32_t* targets,
                                         const rlk_layout_desc_t* layout, const void* rms_gamma,
                                         float* logp, float* lse, float* entropy,
                                         rlk_stream_t stream);

/* Host-only: workspace bytes of rlk_logprob_partials for `num_rows` rows over the vocab range
 * [vocab_begin, vocab_end). */
rlk_status_t rlk_logprob_partials_workspace_size(const rlk_logprob_config_t* config,
                                                 int64_t num_rows, int64_t vocab_begin,
                                                 int64_t vocab_end, size_t* bytes);

/* One vocab shard's local reduction (the "actual vocab range", "target ownership" and "local
 * reduction" of the "Linear logprob" boundary row on the RL-Kernel v0.1.0 summary page, as one
 * rank of its TP4 rollout would compute them): W_shard is bf16 [vocab_end - vocab_begin, H],
 * the rows [vocab_begin, vocab_end) of W_lm; the range must start and end on segment boundaries
 * (multiples of V / S_c), else RLK_ERR_CONTRACT. Writes records[(s - s0) * num_rows + t] for
 * every segment s of the range (s0 = vocab_begin / (V / S_c)) and every row t. */
rlk_status_t rlk_logprob_partials(rlk_logprob_t handle, const void* hidden, const void* W_shard,
                                  int64_t vocab_begin, int64_t vocab_end,
                                  const int32_t* targets, int64_t num_rows,
                                  const void* rms_gamma, rlk_segment_record_t* records,
                                  void* workspace, size_t workspace_bytes, rlk_stream_t stream);

/* Cross-segment merge in the contract's fixed order (the "cross-rank LSE merge" of the "Linear
 * logprob" boundary row and the cross-TP vocab merge of the ROCm fixes list, RL-Kernel v0.1.0
 * summary page): records holds S_c * num_rows records,
 * segment-major (all segments of the vocabulary, gathered from every shard). Writes logp, lse
 * and (with RLK_FLAG_ENTROPY) entropy. status: device uint32 that receives the
 * RLK_DEVICE_STATUS_* bits (OR-ed in), or NULL. */
rlk_status_t rlk_logprob_merge(rlk_logprob_t handle, const rlk_segment_record_t* records,
                               const int32_t* targets, int64_t num_rows, float* logp, float* lse,
                               float* entropy, uint32_t* status, rlk_stream_t stream);

/* Waits for `stream`, then reads the status word a forward left in `workspace`. */
rlk_status_t rlk_logprob_device_status(rlk_logprob_t handle, const void* workspace,
                                       rlk_stream_t stream, uint32_t* flags);

/* Contract id of the handle: every constant that decides a result bit. Two handles give
 * bitwise-identical rows exactly when their contract ids are equal. */
const char* rlk_logprob_contract_id(rlk_logprob_t handle);

/* ---- Backward ----------------------------------------------------------------------------
 * Gradients of L = sum_t grad_logp[t] logp[t] + sum_t grad_entropy[t] entropy[t] (the forward's
 * outputs) with respect to the LM-head input and W_lm. The training side differentiates the
 * recomputed logprob, so the library that fixes the forward provides its backward with fixed
 * numerics too (nxbn.cn blog, §3.3 on the training-side integration; §4.2, an autograd wrapper
 * routing log_softmax's backward to the same library). Contract B1-B3:
 *  B1 dz[t, v] = bf16( (g_t (delta(v = y_t) - p) - gH_t p (z' - lse_t + entropy_t)) inv_tau ),
 *     p = EXP(z' - lse_t), z' recomputed bit for bit as in the forward, in fp32 as written;
 *     rows with y_t < 0 give 0.
 *  B2 grad_hidden = pairwise tree over the vocab segments (in order) of one fp32 MFMA chain per
 *     segment over its vocab indices ascending: bitwise independent of row chunking and equal to
 *     a vocab-sharded computation that merges per-segment partials in that tree.
 *  B3 grad_W = one fp32 MFMA chain over rows ascending (32 at a time, rows padded with zeros to a
 *     multiple of 128), from 0 or, with RLK_BWD_ACCUMULATE, continuing from grad_W's contents;
 *     any row_chunk (a multiple of 128) therefore gives the bits of one pass.
 *  B4 with RLK_FLAG_RMSNORM, B1-B3 run on the RMSNorm's bf16 output (recomputed bit for bit)
 *     and grad_hidden is taken through the RMSNorm (its bf16 rounding passed straight through):
 *     dx = (dy gamma) r - x (c r^3 / H), c = sum (dy gamma) x in the forward's reduction order;
 *     grad_gamma = sum over rows of (dy x) r, as a chain over groups of 128 rows (from 0 or,
 *     with RLK_BWD_ACCUMULATE, from grad_gamma's contents). */
#define RLK_BWD_ACCUMULATE 1u /* grad_W / grad_gamma continue their chains from their contents */

/* Workspace bytes for rlk_logprob_backward with both gradients requested (an upper bound for
 * fewer). row_chunk: 0 (all rows at once) or a positive multiple of 128; rows are processed in
 * chunks of at most that many rows, and of fewer when 2 V_pad bytes per row would pass 2 GiB
 * (V_pad = V rounded up per segment to 128), which changes no result bit. About
 * 2 V_pad rows_per_chunk + 4 S_c rows_per_chunk H bytes, plus about 10 rows_per_chunk H bytes
 * with RLK_FLAG_RMSNORM. */
rlk_status_t rlk_logprob_backward_workspace_size(const rlk_logprob_config_t* config,
                                                 int64_t num_rows, int64_t row_chunk,
                                                 size_t* bytes);

/* hidden bf16 [T, H], W_lm bf16 [V, H], targets int32 [T] (negative = padded): the forward's
 * inputs. lse fp32 [T] and (with grad_entropy) entropy fp32 [T]: the forward's outputs for these
 * rows under this handle. grad_logp fp32 [T]; grad_entropy fp32 [T] or NULL (needs
 * RLK_FLAG_ENTROPY). rms_gamma bf16 [H]: required with RLK_FLAG_RMSNORM, else NULL. Outputs
 * (each optional, at least one): grad_hidden fp32 [T, H], grad_W fp32 [V, H], grad_gamma fp32
 * [H] (RLK_FLAG_RMSNORM only). flags: RLK_BWD_ACCUMULATE (grad_W and grad_gamma continue) or 0.
 * All device pointers 16-byte aligned; the workspace (device, caller-owned) at least
 * rlk_logprob_backward_workspace_size() bytes. Enqueues on stream without synchronizing or
 * allocating. Errors are returned before anything is enqueued. */
rlk_status_t rlk_logprob_backward(rlk_logprob_t handle, const void* hidden, const void* W_lm,
                                  const int32_t* targets, int64_t num_rows,
                                  const void* rms_gamma, const float* lse, const float* entropy,
                                  const float* grad_logp, const float* grad_entropy,
                                  float* grad_hidden, float* grad_W, float* grad_gamma,
                                  uint32_t flags, int64_t row_chunk, void* workspace,
                                  size_t workspace_bytes, rlk_stream_t stream);

/* ---- Backward over vocab shards ------------------------------------------------------------
 * The backward split the way a vocab-parallel (TP) run splits it: each shard computes, for its
 * whole segments, the per-segment dh partials of B2 (before the tree) and its rows of grad_W;
 * the merge then applies B2's segment tree (and, with RLK_FLAG_RMSNORM, B4) to the gathered
 * partials. The result equals rlk_logprob_backward's bit for bit, for any split into shards
 * (the "cross-TP vocab merge" and "fixed rank order" items of the ROCm fixes list on the
 * RL-Kernel v0.1.0 summary page, applied to the gradient). */

/* Host-only: workspace bytes of rlk_logprob_backward_partials for the vocab range
 * [vocab_begin, vocab_end) (whole segments) and row_chunk (as rlk_logprob_backward). */
rlk_status_t rlk_logprob_backward_partials_workspace_size(const rlk_logprob_config_t* config,
                                                          int64_t num_rows, int64_t vocab_begin,
                                                          int64_t vocab_end, int64_t row_chunk,
                                                          size_t* bytes);

/* One vocab shard's backward. W_shard: bf16 rows [vocab_begin, vocab_end) of W_lm (whole
 * segments, else RLK_ERR_CONTRACT). hidden, targets, rms_gamma, lse, entropy, grad_logp and
 * grad_entropy as in rlk_logprob_backward (lse and entropy of the merged forward).
 * dh_parts: fp32 [(vocab_end - vocab_begin) / (V / S_c)][num_rows][H], required: one partial per
 * segment of the shard, w.r.t. the LM-head input (the RMSNorm's output with RLK_FLAG_RMSNORM).
 * grad_W_shard: fp32 [vocab_end - vocab_begin][H] or NULL (RLK_BWD_ACCUMULATE continues it). */
rlk_status_t rlk_logprob_backward_partials(rlk_logprob_t handle, const void* hidden,
                                           const void* W_shard, int64_t vocab_begin,
                                           int64_t vocab_end, const int32_t* targets,
                                           int64_t num_rows, const void* rms_gamma,
                                           const float* lse, const float* entropy,
                                           const float* grad_logp, const float* grad_entropy,
                                           float* dh_parts, float* grad_W_shard, uint32_t flags,
                                           int64_t row_chunk, void* workspace,
                                           size_t workspace_bytes, rlk_stream_t stream);

/* Host-only: workspace bytes of rlk_logprob_backward_merge. */
rlk_status_t rlk_logprob_backward_merge_workspace_size(const rlk_logprob_config_t* config,
                                                       int64_t num_rows, size_t* bytes);

/* Merge of every shard's dh partials: dh_parts fp32 [S_c][num_rows][H], segment-major (all
 * segments of the vocabulary). Writes grad_hidden fp32 [num_rows][H] (through the RMSNorm with
 * RLK_FLAG_RMSNORM, which needs hidden and rms_gamma) and, with RLK_FLAG_RMSNORM, grad_gamma fp32
 * [H] (RLK_BWD_ACCUMULATE continues it). */
rlk_status_t rlk_logprob_backward_merge(rlk_logprob_t handle, const float* dh_parts,
                                        const void* hidden, const void* rms_gamma,
                                        int64_t num_rows, float* grad_hidden, float* grad_gamma,
                                        uint32_t flags, void* workspace, size_t workspace_bytes,
                                        rlk_stream_t stream);

/* Compiler, flags and target the library was built with. */
const char* rlk_build_fingerprint(void);

const char* rlk_status_string(rlk_status_t status);
const char* rlk_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RLK_LOGPROB_H */
