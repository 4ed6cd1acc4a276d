// Internal interface between the host planner (rlk_host.hip) and the kernels (rlk_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rlk_logprob.h"

namespace rlk {

// ---- numeric contract v3 (every constant here decides result bits) ----
constexpr int kVocabTile = 64;    // BV: vocab tile width, tiles start at each segment's start
constexpr int kFoldGroup = 32;    // tiles per sequential group of the segment fold
constexpr int kMaxFoldGroups = 128;  // groups per segment (segments up to 2^18 columns)
constexpr int kMaxSegments = 8;   // S_c in {1, 2, 4, 8}
constexpr int kContractVersion = 3;

// ---- launch shapes (free: they never change a result bit) ----
constexpr int kKStage = 64;       // K elements staged per LDS buffer (2 MFMA steps of 32)

// Arguments of the LM-head tile kernel (one launch = a row range x a range of whole segments).
struct LmheadArgs {
  const uint16_t* hidden;   // bf16 [rows, H], launch row 0
  const uint16_t* W;        // bf16 rows of W_lm starting at global vocab index w_row0
  const int32_t* targets;   // [rows], launch row 0
  float* part_m;            // [tiles][ld] tile maxima, row index already at launch row 0
  float* part_s;            // [tiles][ld] tile sums of exp(z' - m)
  float* part_u;            // [tiles][ld] tile sums of exp(z' - m) (z' - m), or null
  float* tgt;               // [ld] owner-written target logit z'[t, y_t]
  int64_t ld;               // row stride of the partial arrays
  int64_t w_row0;           // global vocab index of W's row 0
  int64_t seg_len;          // V / S_c
  int32_t rows;             // rows in this launch
  int32_t H;
  int32_t tiles_per_seg;    // ceil(seg_len / kVocabTile)
  int32_t seg_begin;        // first segment of this launch
  int32_t n_seg;            // segments in this launch
  int32_t g_base;           // global tile index stored at partial-array row 0
  int32_t n_cu;             // compute units of the device (picks a launch shape only)
  int32_t portable;         // RLK_FLAG_PORTABLE_EXP: software EXP/LOG (C11p)
  float inv_tau;
  uint32_t* queue;          // [kQueueWords] work-queue counters of k_lmhead: zero at launch,
                            // zero again when it ends
  // k_lmhead's item geometry, set by its launcher (all item counts fit 31 bits)
  int32_t q_nvb;            // vocab blocks
  int32_t q_rb;             // row tiles per full band
  int32_t q_nfull;          // full bands
  int32_t q_perf;           // items per queue of a full band: ceil(q_nvb q_rb / 8)
  int32_t q_tail_tt;        // row tiles of the last, partial band (0: none)
  int32_t q_pert;           // items per queue of that band
};
// The workspace's status slot: the status word, then (from word kQueueWord) the queues.
constexpr int kStatusSlotWords = 32;
constexpr int kQueueWord = 16;
constexpr int kQueueWords = 9;
// A block of the LM-head kernels covers a run of consecutive tiles of one segment (4 tiles,
// 256 columns, for the MFMA-bound shapes; 3 tiles, 192 columns, for launches of few rows) and
// a run of rows; each wave of it owns whole tiles, so every tile's reductions stay in one wave.

struct MergeArgs {
  const rlk_segment_record_t* rec;  // [n_seg][rec_ld], all segments of the vocabulary
  const int32_t* targets;
  float* logp;
  float* lse;
  float* entropy;           // null without entropy
  uint32_t* status;         // null allowed
  int64_t rec_ld;
  int64_t seg_len;
  int64_t vocab;
  int32_t rows;
  int32_t n_seg;
  int32_t portable;
};

struct FoldArgs {
  const float* part_m;
  const float* part_s;
  const float* part_u;      // null without entropy
  const float* tgt;
  const int32_t* targets;
  rlk_segment_record_t* rec;  // [n_seg][rec_ld]
  int64_t ld;
  int64_t rec_ld;
  int64_t seg_len;
  int32_t rows;
  int32_t tiles_per_seg;
  int32_t seg_begin;
  int32_t n_seg;
  int32_t g_base;
  int32_t portable;
  // Fused merge: null, or one counter per 64-row block of the launch (zero on entry, zero again
  // on exit); the fold of a row block's last segment then also writes mg's outputs for it. Needs
  // the launch to cover every segment of the vocabulary (mg.rec = rec).
  uint32_t* done;
  MergeArgs mg;
};

struct RmsArgs {
  const uint16_t* x;        // bf16 [rows, H]
  const uint16_t* gamma;    // bf16 [H]
  uint16_t* y;              // bf16 [rows, H]
  int32_t rows;
  int32_t H;
  float inv_H;              // fl32(1/H)
  float eps;
  int32_t portable;         // RSQ as a correctly rounded 1/sqrt (C11p)
};

// ---- backward ----
constexpr int kBwdKPad = 128;  // K of the backward GEMMs (vocab per segment, rows) padded to this

// NT GEMM tile kernel of the backward: acc[m, n] = sum_k A[m, k] B[n, k] (bf16, fp32 MFMA chain,
// K ascending from +0 or from the stored output), then one of two epilogues.
//  DZ:  m = segment-padded vocab position (M = S_c Lp; A row m is W row v(m)), B = LM-head input
//       rows (n = row t), K = H. Writes the bf16 gradient of the tempered logits' loss (B1) to
//       dz[t][m], zeros at padding positions.
//  OUT: writes C[row(n) * ldc + m] in fp32 (dh: m = h, n = t; dW: m = h, n = padded vocab row).
//       A is K-major (row k of A holds the M indices: W for dh, the hidden rows for dW; ka_rows
//       valid K rows, lda its row stride); B is K-contiguous (dz rows, dh) or K-major (dz, dW;
//       kb_rows valid K rows). K-major rows past the valid ones read as zeros.
// col(v) / row(n) is the segment-padded vocab layout: v = s seg_len + c <-> s seg_pad + c.
struct GemmArgs {
  const uint16_t* A;
  int64_t lda;
  const uint16_t* B;
  int64_t ldb;
  int32_t M, N, K;          // K: a multiple of kBwdKPad
  int64_t seg_len;          // L = V / S_c (segment-padded vocab layout)
  int64_t seg_pad;          // Lp = L rounded up to kBwdKPad
  // OUT
  float* C;
  int64_t ldc;
  int64_t c_batch;          // C offset per batch (one vocab segment per batch for dh)
  int64_t a_batch, b_batch; // A / B offsets per batch
  int32_t accumulate;       // start the chain from C's stored values
  int32_t map_rows;         // OUT rows n are segment-padded vocab rows (skip padding rows)
  int64_t ka_rows, kb_rows; // valid K rows of a K-major A / B
  // DZ
  const int32_t* targets;   // [rows]
  const float* lse;         // forward lse [rows]
  const float* ent;         // forward entropy [rows] (with grad_ent)
  const float* g;           // dL/dlogp [rows]
  const float* gH;          // dL/dentropy [rows] or null
  uint16_t* dz;             // bf16 [rows][S_c Lp]
  int64_t lddz;
  int64_t v_base;           // global vocab index of position 0 (a shard's first row)
  float inv_tau;
  int32_t portable;
  // persistent launch: work queues ([kQueueWords] counters, zero at launch, left zero) and the
  // item geometry (queue_setup over the A tiles x (batch, B tile) pairs)
  uint32_t* queue;
  int32_t n_cu;
  int32_t n_bt;             // B tiles per batch
  int32_t q_nvb, q_rb, q_nfull, q_perf, q_tail_tt, q_pert;
};


// B4: the final RMSNorm's backward, one wave per row. dx (optional) and r (optional) per row.
struct RmsBwdArgs {
  const uint16_t* x;        // bf16 [rows, H] (the RMSNorm's input)
  const uint16_t* gamma;    // bf16 [H]
  const float* dy;          // fp32 [rows, H]: gradient w.r.t. the RMSNorm's output
  float* dx;                // fp32 [rows, H] or null
  float* r;                 // fp32 [rows] or null: the rows' 1/rms (C12 bits)
  int32_t rows;
  int32_t H;
  float inv_H;
  float eps;
  int32_t portable;
};
constexpr int kGammaGroup = 128;  // rows per sequential group of the dgamma sum (B4)

hipError_t launch_rmsnorm_bwd(const RmsBwdArgs& a, hipStream_t s);
// P[q][k] = sum over rows t of group q (kGammaGroup rows, ascending, from +0) of
// (dy[t][k] x[t][k]) r[t]; then dgamma[k] = chain over q ascending from 0 or dgamma[k].
hipError_t launch_dgamma(const float* dy, const uint16_t* x, const float* r, float* P, int rows,
                         int H, float* dgamma, bool accumulate, hipStream_t s);

hipError_t launch_gemm_dz(const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm_out(const GemmArgs& a, int batches, bool b_trans, hipStream_t s);
// fp32 zeros over n elements (a fill kernel: usable under graph capture)
hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t s);
// out[i] = balanced pairwise tree over s < nseg of part[s * stride + i] (nseg in 1, 2, 4, 8)
hipError_t launch_seg_tree(const float* part, int64_t stride, int nseg, float* out, int64_t n,
                           hipStream_t s);

// Token-tile widths the LM-head kernel can be forced to (0 = chosen per launch).
bool token_tile_supported(int bt);

hipError_t launch_lmhead(const LmheadArgs& a, int token_tile, bool entropy, hipStream_t s);
hipError_t launch_fold(const FoldArgs& a, bool entropy, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, bool entropy, hipStream_t s);
hipError_t launch_rmsnorm(const RmsArgs& a, hipStream_t s);
// Zeroes the status slot (status word and LM-head work queues) and n_done fused-merge counters.
hipError_t launch_clear_status(uint32_t* status, uint32_t* done, int64_t n_done, hipStream_t s);

}  // namespace rlk
