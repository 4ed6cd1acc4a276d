// HIP kernels of the backward of the strict-path selected-token logprob, for gfx950 (MI355X) only.
//
// The training side differentiates the recomputed logprob, so the library that fixes the forward
// also provides its backward, with the same care for fixed numerics (nxbn.cn blog, §3.3 on the
// training-side integration and §4.2, whose autograd wrapper hands log_softmax's backward to the
// same kernel library). The loss seen by the path is L = sum_t g_t logp_t + sum_t gH_t entropy_t.
// Backward contract, on top of the forward's C1-C12:
//
//  B1 dz. For a row t with y_t >= 0 and a vocab index v: z' is computed as in C1-C2 (the
//     forward's bits); p = EXP(z' - lse_t) with the forward's lse_t; d = 1 - p if v = y_t, else
//     -p; q = g_t d; with gH: q = q - gH_t (p ((z' - lse_t) + ent_t)); q = q inv_temperature
//     (skipped when it is 1.0f); dz = bf16_rne(q). Rows with y_t < 0 give dz = +0. dz is the
//     operand of the two bf16 GEMMs below, hence its bf16 materialization (the one rounding
//     point besides fp32 arithmetic).
//  B2 dh, the gradient with respect to the LM-head input. Per vocab segment s (C3's split):
//     D_s[t, k] = one fp32 v_mfma_f32_16x16x32_bf16 chain over the segment's vocab indices
//     ascending, 32 at a time, from +0; each segment is padded with zero columns to a multiple
//     of 128, which adds exact zeros. dh = balanced pairwise tree of the D_s in segment order
//     (the C9 tree), so a vocab-sharded run reproduces it.
//  B3 dW[v, k] = one fp32 MFMA chain over the rows t ascending, 32 at a time, from +0 or from
//     the stored dW (accumulate); rows are padded with zeros to a multiple of 128. Row chunks of
//     a multiple of 128 rows continue the chain, so chunked and one-pass runs give the same bits.
//     With the final RMSNorm, B1-B3 run on its bf16 output y (C12's bits, recomputed).
//  B4 RMSNorm (optional). dy = B2's gradient w.r.t. y; the bf16 rounding of y is passed straight
//     through. Per row: c = sum_k (dy_k gamma_k) x_k and ss = sum_k x_k^2, both in C12's order
//     (lane l takes the 8-element groups l, l+64, .. sequentially, then the xor butterfly 32 ..
//     1); r = RSQ(ss fl32(1/H) + eps) exactly as in C12; a = ((r r) r) fl32(1/H);
//     dx_k = (dy_k gamma_k) r - x_k (c a). dgamma_k = a chain over groups of 128 rows ascending,
//     from 0 or the stored dgamma, of P_q = sum over the group's rows ascending, from +0, of
//     (dy_tk x_tk) r_t; row chunks of a multiple of 128 rows continue it.
//
// Layout: dz [rows][S_c Lp] (in the caller's workspace) holds vocab index v = s L + c at the
// segment-padded position s Lp + c (L = V / S_c, Lp = L rounded up to 128), with zeros at the
// padding positions; the dz kernel runs over the padded positions, so it writes those zeros.
// All three GEMMs run on the forward's K loop (nt_mainloop). dh reads W as it is stored (K =
// vocab index is its row index) and dW reads the hidden rows and dz as they are stored (K = row),
// through the K loop's transposed staging (ds_read_b64_tr_b16): nothing is transposed in memory.

#include <algorithm>
#include <utility>

#include "rlk_device.h"
#include "rlk_queue.h"

namespace rlk {

namespace {

// Block tile of the backward GEMMs: 256 A rows x 256 B rows, 8 waves (2 along A, 4 along B),
// a wave tile of 128 x 64, the shape of the forward's main kernel.
constexpr int kGVW = 2, kGTW = 4, kGNTB = 2;
constexpr int kGWaves = kGVW * kGTW;
constexpr int kGBM = 256;                  // A rows per block
constexpr int kGBN = 32 * kGNTB * kGTW;    // B rows per block (256)
constexpr int kGVB16 = kGBM / 16 / kGVW;   // A blocks of 16 per wave (8)
constexpr int kGNB16 = 2 * kGNTB;          // B blocks of 16 per wave (4)
constexpr int kGWI = kGBM / 8 / kGWaves;   // A DMA instructions per wave per stage
constexpr int kGHI = kGBN / 8 / kGWaves;   // B DMA instructions per wave per stage

template <int... Is, class F>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, Is...>, F&& f) {
  (f(std::integral_constant<int, Is>{}), ...);
}
// f(integral_constant<int, 0>) .. f(integral_constant<int, N - 1>), in order
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(std::make_integer_sequence<int, N>{}, f);
}

struct GTile {
  int m0, mrows, n0, nrows;
};

// Item -> (A tile, batch, B tile). A launch's items are the A tiles x (batch, B tile) pairs,
// handed out by per-XCD work queues (rlk_queue.h) in the forward's XCD-aware order: each XCD
// walks a contiguous range of items, a group of 8 A tiles at a time across the B side.
__device__ __forceinline__ void set_gtile(const GemmArgs& a, int vb, int tt, GTile& t, int& yb) {
  const int y = tt / a.n_bt;
  const int nt = tt - y * a.n_bt;
  yb = uni(y);
  t.m0 = uni(vb * kGBM);
  t.mrows = uni(min(kGBM, a.M - vb * kGBM));
  t.n0 = uni(nt * kGBN);
  t.nrows = uni(min(kGBN, a.N - nt * kGBN));
}

// Hands out one item of queue x (the count of items handed out from it before).
__device__ __forceinline__ uint32_t gclaim(uint32_t* q, int x) {
  return __hip_atomic_fetch_add(q + x, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The item behind claim count c of queue (xq + qi) mod 8; a drained queue moves the block on to
// the next queue, and false means that all eight are drained (at most eight claims).
__device__ __forceinline__ bool gnext(const GemmArgs& a, int xq, int& qi, uint32_t c, int& vb,
                                      int& tt) {
  while (true) {
    if (queue_item(a, (xq + qi) & (kQueues - 1), c, vb, tt)) return true;
    if (++qi == kQueues) return false;
    c = gclaim(a.queue, (xq + qi) & (kQueues - 1));
  }
}

// Output row of tile B row nn (OUT epilogue), or null for a row past the tile or a padding row
// of the segment-padded vocab layout. 32-bit index math: B rows are below 2^31.
__device__ __forceinline__ float* out_row(const GemmArgs& a, float* C, const GTile& t, int nn) {
  if (nn >= t.nrows) return nullptr;
  const uint32_t n = (uint32_t)(t.n0 + nn);
  uint32_t row = n;
  if (a.map_rows) {
    const uint32_t Lp = (uint32_t)a.seg_pad, L = (uint32_t)a.seg_len;
    const uint32_t sg = n / Lp;
    const uint32_t c = n - sg * Lp;
    if (c >= L) return nullptr;
    row = sg * L + c;
  }
  return C + (int64_t)row * a.ldc;
}

// Store shape of the epilogues. The MFMA result gives lane l = 16 g + r (r = l & 15) the row r of
// a B block and 16 bytes of A block i at 16 i + 4 g; stored as is, one store instruction writes
// 16 rows x 64 bytes (half cache lines), and a CU's store path takes about as long per line
// touched as per full line (measured: 34 GB/s per CU against ~95 GB/s for 8 rows x 128 bytes).
// So the data of two A blocks is regrouped across lanes first: with Y's rows rotated by 8 within
// each 16 lanes (DPP row_ror:8), lanes r < 8 hold X of row r and Y of row r + 8, lanes r >= 8 the
// reverse, and two store instructions write rows 0-7 and rows 8-15 as whole 128-byte lines.
__device__ __forceinline__ uint32_t ror8(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x128, 0xF, 0xF, false);
}

// One B1 value before its rounding to bf16.
template <bool ENTG, bool TEMP, bool PORT>
__device__ __forceinline__ float dz_q(float acc, int v, int y, float g, float l, float gh, float e,
                                      float inv_tau) {
  const float zp = TEMP ? acc * inv_tau : acc;
  const float p = EXP<PORT>(zp - l);
  const float d = (v == y) ? 1.0f - p : -p;
  float q = g * d;
  if constexpr (ENTG) q = q - gh * (p * ((zp - l) + e));
  if constexpr (TEMP) q = q * inv_tau;
  return q;
}

// Two values rounded to bf16 (to nearest even, a NaN kept quiet with its top payload bits), as
// one word: gfx950's v_cvt_pk_bf16_f32, whose results equal that rounding written out in integer
// arithmetic for every one of the 2^32 fp32 inputs (checked exhaustively on the device).
__device__ __forceinline__ uint32_t pack_bf16(float x0, float x1) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const f2 x = {x0, x1};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, b2));
}

// Staging of one tile: per-lane DMA offsets of stage 0 and the operands' buffer descriptors.
// Rows past the tile are clamped to its last row, as in the forward. DZ runs over the
// segment-padded vocab positions: tile row m reads W row v(m), a padding position the last row
// of its segment (its result is replaced by 0). v(m) never decreases, and the tile's real rows
// are consecutive in W, so one descriptor from v(first) covers them.
template <int EPI, bool ATR, bool BTR>
__device__ __forceinline__ void gemm_stage(const GemmArgs& a, const GTile& t, int yb, int wave,
                                           int lane, uint32_t (&ago)[kGWI],
                                           uint32_t (&bgo)[kGHI], __amdgpu_buffer_rsrc_t& ra,
                                           __amdgpu_buffer_rsrc_t& rb) {
  const uint16_t* __restrict__ Bt =
      BTR ? a.B + yb * a.b_batch + t.n0 : a.B + yb * a.b_batch + (int64_t)t.n0 * a.ldb;
  const uint16_t* __restrict__ At;
  int64_t a_rows;  // rows the A descriptor spans
  if constexpr (EPI == 0) {
    const uint32_t L = (uint32_t)a.seg_len, Lp = (uint32_t)a.seg_pad;
    auto vrow = [&](uint32_t m) {
      const uint32_t sg = m / Lp;
      return sg * L + min(m - sg * Lp, L - 1);
    };
    const uint32_t vf = (uint32_t)uni((int)vrow((uint32_t)t.m0));
    const uint32_t vl = (uint32_t)uni((int)vrow((uint32_t)(t.m0 + t.mrows - 1)));
    At = a.A + (int64_t)vf * a.lda;
    a_rows = (int64_t)(vl - vf) + 1;
#pragma unroll
    for (int q = 0; q < kGWI; ++q) {
      const int r = 8 * (q * kGWaves + wave) + (lane >> 3);
      const int c = (lane & 7) ^ swz(r);
      const uint32_t v = vrow((uint32_t)(t.m0 + min(r, t.mrows - 1))) - vf;
      ago[q] = (uint32_t)(((int64_t)v * a.lda + c * 8) * 2);
    }
  } else if constexpr (ATR) {
    At = a.A + yb * a.a_batch + t.m0;
    a_rows = 0;
  } else {
    At = a.A + yb * a.a_batch + (int64_t)t.m0 * a.lda;
    a_rows = t.mrows;
#pragma unroll
    for (int q = 0; q < kGWI; ++q) {
      const int r = 8 * (q * kGWaves + wave) + (lane >> 3);
      const int c = (lane & 7) ^ swz(r);
      ago[q] = (uint32_t)(((int64_t)min(r, t.mrows - 1) * a.lda + c * 8) * 2);
    }
  }
  // A K-major (transposed) operand is staged 64 K rows x 256 indices per stage: DMA instruction q
  // of this wave fills rows 2 (q NWAVES + wave) and the next, lane l slot l & 31 of its row,
  // with the piece the swizzle puts there. Its descriptor spans the valid K rows only (and ends
  // at the array's last element), so padding rows read as zeros.
  auto tr_offsets = [&](uint32_t* go, int64_t ld) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 2 * (q * kGWaves + wave) + (lane >> 5);
      const int pc = (lane & 31) ^ tswz(r);
      go[q] = (uint32_t)(((int64_t)r * ld + pc * 8) * 2);
    }
  };
  auto tr_bytes = [&](int64_t krows, int64_t ld, int i0) {
    return (int)(((krows - 1) * ld + min<int64_t>(256, ld - i0)) * 2);
  };
  if constexpr (ATR) {
    static_assert(kGWI == 4, "64 K rows x 512 bytes per stage = 4 DMA instructions per wave");
    tr_offsets(ago, a.lda);
  }
  if constexpr (BTR) {
    static_assert(kGHI == 4, "64 K rows x 512 bytes per stage = 4 DMA instructions per wave");
    tr_offsets(bgo, a.ldb);
  } else {
#pragma unroll
    for (int q = 0; q < kGHI; ++q) {
      const int r = 8 * (q * kGWaves + wave) + (lane >> 3);
      const int c = (lane & 7) ^ swz(r);
      bgo[q] = (uint32_t)(((int64_t)min(r, t.nrows - 1) * a.ldb + c * 8) * 2);
    }
  }
  ra = ATR ? make_rsrc(At, tr_bytes(a.ka_rows, a.lda, t.m0))
           : make_rsrc(At, (int)(((a_rows - 1) * a.lda + a.K) * 2));
  rb = BTR ? make_rsrc(Bt, tr_bytes(a.kb_rows, a.ldb, t.n0))
           : make_rsrc(Bt, (int)(((int64_t)(t.nrows - 1) * a.ldb + a.K) * 2));
}

// DMA of K stage kc of both operands into (la, lb), as the K loop issues it; sa / sb: bytes
// from one K stage to the next of a K-major operand.
template <bool ATR, bool BTR>
__device__ __forceinline__ void gemm_issue(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                           const uint32_t (&ago)[kGWI],
                                           const uint32_t (&bgo)[kGHI], int kc, uint8_t* la,
                                           uint8_t* lb, int wave, uint32_t sa, uint32_t sb) {
  const uint32_t so = (uint32_t)kc * kRowBytes;
  const uint32_t soa = ATR ? (uint32_t)kc * sa : so;
  const uint32_t sob = BTR ? (uint32_t)kc * sb : so;
#pragma unroll
  for (int q = 0; q < kGWI; ++q) dma16(ra, la + 8 * (q * kGWaves + wave) * kRowBytes, ago[q], soa);
#pragma unroll
  for (int q = 0; q < kGHI; ++q) dma16(rb, lb + 8 * (q * kGWaves + wave) * kRowBytes, bgo[q], sob);
}

// The B1 inputs of this lane's rows (lane & 15 of each of the wave's B blocks).
struct DzRows {
  int y[kGNB16];
  float g[kGNB16], l[kGNB16], h[kGNB16], e[kGNB16];
};

template <bool ENTG>
__device__ __forceinline__ void dz_rows(const GemmArgs& a, const GTile& t, int wt, int ln,
                                        DzRows& r) {
#pragma unroll
  for (int j = 0; j < kGNB16; ++j) {
    const int nn = 16 * (wt * kGNB16 + j) + (ln & 15);
    const bool ok = nn < t.nrows;
    const int64_t n = t.n0 + (ok ? nn : 0);
    r.y[j] = ok ? a.targets[n] : -1;
    r.g[j] = a.g[n];
    r.l[j] = a.lse[n];
    r.h[j] = ENTG ? a.gH[n] : 0.0f;
    r.e[j] = ENTG ? a.ent[n] : 0.0f;
  }
}

// B1 on the result registers: lane l holds the token row l & 15 of each B block and 4
// consecutive vocab positions of each A block, which become 4 bf16 (8 bytes). A group of four A
// blocks (64 positions = 128 bytes of a dz row) is regrouped to 16 bytes per lane in two steps:
// v_permlane16_swap exchanges 16-lane rows 1 <-> 0 and 3 <-> 2 between blocks (i, i+1), so that
// lane 16 g + r holds positions 8 (g >> 1) .. +7 of block i + (g & 1) (P; likewise Q for blocks
// i+2, i+3), then the ror8 step above pairs token rows r and r + 8. The epilogues index the
// accumulators with compile-time constants (static_for): a runtime index would move them to
// scratch.
template <bool ENTG, bool TEMP, bool PORT>
__device__ __forceinline__ void dz_epilogue(const GemmArgs& a, f32x4 (&acc)[kGVB16][kGNB16],
                                            const DzRows& rw, const GTile& t, int wv, int wt,
                                            int ln) {
  const int r = ln & 15, g = ln >> 4;
  const bool lo = r < 8;
  const uint32_t L = (uint32_t)a.seg_len, Lp = (uint32_t)a.seg_pad;
  const uint32_t wb = (uint32_t)(t.m0 + 16 * wv * kGVB16);  // the wave's first position
  const uint32_t cb = wb + 4 * g;                            // this lane's position in block 0
  // position of this lane's 16 bytes after the regrouping, in the group's first block pair
  const uint32_t cp = wb + 16 * (g & 1) + 8 * (g >> 1);
  static_for<kGNB16>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    const int nn_a = 16 * (wt * kGNB16 + j) + (r & 7);  // rows of the two stores
    const bool ok_a = nn_a < t.nrows, ok_b = nn_a + 8 < t.nrows;
    uint16_t* const da = a.dz + (t.n0 + (int64_t)nn_a) * a.lddz;
    uint16_t* const db = da + 8 * a.lddz;
    static_for<kGVB16 / 4>([&](auto gc) {
      constexpr int i0 = 4 * decltype(gc)::value;
      uint32_t w[4][2];  // the lane's 4 bf16 of blocks i0 .. i0+3
      static_for<4>([&](auto qc) {
        constexpr int q = decltype(qc)::value;
        const uint32_t col0 = cb + 16 * (i0 + q);
        const uint32_t sg = col0 / Lp;
        const uint32_t c0 = col0 - sg * Lp;           // position inside the segment
        const int v0 = (int)(a.v_base + sg * L + c0);  // vocab index of col0 when c0 < L
        // padding positions and rows without a target give +0
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          x[e] = c0 + e < L ? dz_q<ENTG, TEMP, PORT>(acc[i0 + q][j][e], v0 + e, rw.y[j], rw.g[j],
                                                     rw.l[j], rw.h[j], rw.e[j], a.inv_tau)
                            : 0.0f;
        const uint32_t ym = 0u - (uint32_t)(rw.y[j] >= 0);
        w[q][0] = pack_bf16(x[0], x[1]) & ym;
        w[q][1] = pack_bf16(x[2], x[3]) & ym;
      });
      uint32_t P[4], Q[4];
      {
        const auto s0 = __builtin_amdgcn_permlane16_swap(w[0][0], w[1][0], false, false);
        const auto s1 = __builtin_amdgcn_permlane16_swap(w[0][1], w[1][1], false, false);
        const auto s2 = __builtin_amdgcn_permlane16_swap(w[2][0], w[3][0], false, false);
        const auto s3 = __builtin_amdgcn_permlane16_swap(w[2][1], w[3][1], false, false);
        P[0] = s0[0]; P[1] = s1[0]; P[2] = s0[1]; P[3] = s1[1];
        Q[0] = s2[0]; Q[1] = s3[0]; Q[2] = s2[1]; Q[3] = s3[1];
      }
      u32x4 pv, zv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pv[e] = P[e];
        zv[e] = ror8(Q[e]);
      }
      const uint32_t c_p = cp + 16 * i0;  // P's positions; Q's are 32 further
      const uint32_t ca = lo ? c_p : c_p + 32, cbb = lo ? c_p + 32 : c_p;
      if (ok_a && (int)ca < a.M) *(u32x4*)(da + ca) = lo ? pv : zv;
      if (ok_b && (int)cbb < a.M) *(u32x4*)(db + cbb) = lo ? zv : pv;
    });
  });
}

// OUT: fp32, A blocks (i, i+1) regrouped as above into two stores of 8 rows x 128 bytes.
__device__ __forceinline__ void out_store(const GemmArgs& a, f32x4 (&acc)[kGVB16][kGNB16],
                                          const GTile& t, int yb, int wv, int wt, int ln) {
  float* C = a.C + yb * a.c_batch;
  const int r = ln & 15, g = ln >> 4;
  const bool lo = r < 8;
  const int mb = t.m0 + 16 * wv * kGVB16 + 4 * g;  // this lane's column in A block 0
  static_for<kGNB16>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    const int nn_a = 16 * (wt * kGNB16 + j) + (r & 7);
    float* const ra = out_row(a, C, t, nn_a);
    float* const rb = out_row(a, C, t, nn_a + 8);
    static_for<kGVB16 / 2>([&](auto pc) {
      constexpr int i0 = 2 * decltype(pc)::value;
      const f32x4 X = acc[i0][j];
      f32x4 Z;
#pragma unroll
      for (int e = 0; e < 4; ++e) Z[e] = __uint_as_float(ror8(__float_as_uint(acc[i0 + 1][j][e])));
      const int c = mb + 16 * i0;  // X's columns; Z's are 16 further
      const int ca = lo ? c : c + 16, cbb = lo ? c + 16 : c;
      if (ra && ca < a.M) *(f32x4*)(ra + ca) = lo ? X : Z;
      if (rb && cbb < a.M) *(f32x4*)(rb + cbb) = lo ? Z : X;
    });
  });
}

// ACC: the stored values as the chain's start, in the MFMA result layout.
__device__ __forceinline__ void out_load(const GemmArgs& a, f32x4 (&acc)[kGVB16][kGNB16],
                                         const GTile& t, int yb, int wv, int wt, int ln) {
  float* C = a.C + yb * a.c_batch;
  static_for<kGNB16>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    const float* crow = out_row(a, C, t, 16 * (wt * kGNB16 + j) + (ln & 15));
    if (!crow) return;
    const int mb = t.m0 + 16 * wv * kGVB16 + 4 * (ln >> 4);
    static_for<kGVB16>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if (mb + 16 * i < a.M) acc[i][j] = *(const f32x4*)(crow + mb + 16 * i);
    });
  });
}

// The backward's NT GEMM kernel (see GemmArgs). EPI 0 = DZ, 1 = OUT.
// Persistent, as the forward's LM-head kernel: one block per CU takes items from its XCD's work
// queue, then from the other XCDs' queues. Once every wave is past an item's last fragment read,
// the first two K stages of the next item are issued, and only then does the item's epilogue
// compute and store its results, so the next item's loads overlap them. Which block computes an
// item never changes its arithmetic, so the bits do not depend on the schedule.
template <int EPI, bool ENTG, bool TEMP, bool PORT, bool ACC, bool ATR, bool BTR>
__global__ void __launch_bounds__(64 * kGWaves) k_gemm(const GemmArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds_a0[kGBM * kRowBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_a1[kGBM * kRowBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_b0[kGBN * kRowBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_b1[kGBN * kRowBytes];
  // the block's next item (A tile, batch x B tile), -1 when every queue is drained, and the
  // queue offset of its claims; written by thread 0, read after barriers
  __shared__ int s_next[2];
  __shared__ int s_qi;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wv = wave % kGVW;
  const int wt = wave / kGVW;
  const bool leader = tid == 0;
  const int nk = a.K / kKStage;
  const uint32_t sa = (uint32_t)(64 * a.lda * 2), sb = (uint32_t)(64 * a.ldb * 2);
  // this XCD's queue: the XCC_ID hardware register (the id is bits 3:0)
  auto xcc_queue = []() { return (int)(__builtin_amdgcn_s_getreg((31 << 11) | 20) & (kQueues - 1)); };
  // The arguments again from the kernel-argument segment, by scalar loads through a pointer the
  // compiler cannot see through: what the item boundary needs is loaded there instead of held in
  // scalar registers across the K loop.
  typedef const __attribute__((address_space(4))) GemmArgs* kargs_t;
  auto args = []() -> const GemmArgs& {
    uint64_t p = (uint64_t)__builtin_amdgcn_kernarg_segment_ptr();
    __asm__ volatile("" : "+s"(p));
    return *(const GemmArgs*)(kargs_t)p;
  };
  uint32_t pend = 0;  // thread 0: claim count in flight for the next item

  if (leader) {
    const int xq = xcc_queue();
    int qi = 0, vb = -1, tt = 0;
    if (!gnext(a, xq, qi, gclaim(a.queue, xq), vb, tt)) vb = -1;
    s_next[0] = vb;
    s_next[1] = tt;
    s_qi = qi;
  }
  __syncthreads();
  if (uni(s_next[0]) >= 0) {
    GTile t;
    int yb;
    set_gtile(a, uni(s_next[0]), uni(s_next[1]), t, yb);
    uint32_t ago[kGWI], bgo[kGHI];
    __amdgpu_buffer_rsrc_t ra, rb;
    gemm_stage<EPI, ATR, BTR>(a, t, yb, wave, lane, ago, bgo, ra, rb);
    gemm_issue<ATR, BTR>(ra, rb, ago, bgo, 0, lds_a0, lds_b0, wave, sa, sb);
    gemm_issue<ATR, BTR>(ra, rb, ago, bgo, 1, lds_a1, lds_b1, wave, sa, sb);
    if (leader) pend = gclaim(a.queue, (xcc_queue() + s_qi) & (kQueues - 1));
    while (true) {
      f32x4 acc[kGVB16][kGNB16];
#pragma unroll
      for (int i = 0; i < kGVB16; ++i)
#pragma unroll
        for (int j = 0; j < kGNB16; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.0f;
      if constexpr (EPI == 1 && ACC) out_load(args(), acc, t, yb, wv, wt, lane);
      auto resolve = [&]() {
        if (leader) {
          int qi = s_qi, nv = -1, nt = 0;
          if (!gnext(args(), xcc_queue(), qi, pend, nv, nt)) nv = -1;
          s_next[0] = nv;
          s_next[1] = nt;
          s_qi = qi;
        }
      };
      nt_mainloop_x<kGWaves, kGVB16, kGNB16, kGWI, kGHI, ATR, BTR, true>(
          acc, lds_a0, lds_a1, lds_b0, lds_b1, ra, rb, ago, bgo, nk, wave, lane, wv, wt, sa, sb,
          resolve);
      __syncthreads();
      const GemmArgs& b = args();
      // an opaque copy of the lane id: what the epilogue derives from it is computed here, not
      // hoisted out of the item loop and held across the K loop
      int ln = lane;
      __asm__ volatile("" : "+v"(ln));
      // B1's row inputs are loaded before the next item's DMAs, so that waiting for them does
      // not wait for those
      DzRows rw;
      if constexpr (EPI == 0) dz_rows<ENTG>(b, t, wt, ln, rw);
      const int nv = uni(s_next[0]);
      if (nv >= 0) {
        GTile tn;
        int yn;
        set_gtile(b, nv, uni(s_next[1]), tn, yn);
        gemm_stage<EPI, ATR, BTR>(b, tn, yn, wave, ln, ago, bgo, ra, rb);
        gemm_issue<ATR, BTR>(ra, rb, ago, bgo, 0, lds_a0, lds_b0, wave, sa, sb);
        gemm_issue<ATR, BTR>(ra, rb, ago, bgo, 1, lds_a1, lds_b1, wave, sa, sb);
        if (leader) pend = gclaim(b.queue, (xcc_queue() + s_qi) & (kQueues - 1));
      }
      if constexpr (EPI == 1) out_store(b, acc, t, yb, wv, wt, ln);
      else dz_epilogue<ENTG, TEMP, PORT>(b, acc, rw, t, wv, wt, ln);
      if (nv < 0) break;
      // the next item again from the queue's answer, rather than held across the epilogue
      __asm__ volatile("" ::: "memory");
      set_gtile(args(), uni(s_next[0]), uni(s_next[1]), t, yb);
    }
  }
  // the last block of the launch to get here resets the queues for the next launch
  if (leader && gclaim(a.queue, kQueues) == gridDim.x - 1) {
    for (int x = 0; x <= kQueues; ++x)
      __hip_atomic_exchange(a.queue + x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

__global__ void k_zero_f32(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.0f;
}

template <int NS>
__global__ void k_seg_tree(const float* part, int64_t stride, float* out, int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * blockDim.x) {
    f32x4 v[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) v[s] = *(const f32x4*)(part + s * stride + 4 * i);
    f32x4 o;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float w[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s) w[s] = v[s][r];
      o[r] = tree_sum<NS>(w);
    }
    *(f32x4*)(out + 4 * i) = o;
  }
}

__global__ void __launch_bounds__(256) k_rmsnorm_bwd(const RmsBwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const uint16_t* __restrict__ x = a.x + (int64_t)row * a.H;
  const float* __restrict__ dy = a.dy + (int64_t)row * a.H;
  const int npieces = a.H / 8;
  float ss = 0.0f, c = 0.0f;
  for (int p = lane; p < npieces; p += 64) {
    const u32x4 v = *(const u32x4*)(x + p * 8);
    const u32x4 g = *(const u32x4*)(a.gamma + p * 8);
    const f32x4 d0 = *(const f32x4*)(dy + p * 8);
    const f32x4 d1 = *(const f32x4*)(dy + p * 8 + 4);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float xl = bf16_to_f32(v[w] & 0xffffu), xh = bf16_to_f32(v[w] >> 16);
      const float gl = bf16_to_f32(g[w] & 0xffffu), gh = bf16_to_f32(g[w] >> 16);
      const float dl = w < 2 ? d0[2 * w] : d1[2 * w - 4];
      const float dh = w < 2 ? d0[2 * w + 1] : d1[2 * w - 3];
      ss = ss + xl * xl;
      ss = ss + xh * xh;
      c = c + (dl * gl) * xl;
      c = c + (dh * gh) * xh;
    }
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    ss = ss + __shfl_xor(ss, d);
    c = c + __shfl_xor(c, d);
  }
  const float v = ss * a.inv_H + a.eps;
  const float r = a.portable ? p_rsq(v) : c_rsq(v);
  const float b = c * (((r * r) * r) * a.inv_H);
  if (a.r && lane == 0) a.r[row] = r;
  if (!a.dx) return;
  float* __restrict__ dx = a.dx + (int64_t)row * a.H;
  for (int p = lane; p < npieces; p += 64) {
    const u32x4 v8 = *(const u32x4*)(x + p * 8);
    const u32x4 g = *(const u32x4*)(a.gamma + p * 8);
    const f32x4 d0 = *(const f32x4*)(dy + p * 8);
    const f32x4 d1 = *(const f32x4*)(dy + p * 8 + 4);
    f32x4 o0, o1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t wx = v8[e >> 1], wg = g[e >> 1];
      const float xv = bf16_to_f32((e & 1) ? (wx >> 16) : (wx & 0xffffu));
      const float gv = bf16_to_f32((e & 1) ? (wg >> 16) : (wg & 0xffffu));
      const float dv = e < 4 ? d0[e] : d1[e - 4];
      const float o = (dv * gv) * r - xv * b;
      if (e < 4) o0[e] = o;
      else o1[e - 4] = o;
    }
    *(f32x4*)(dx + p * 8) = o0;
    *(f32x4*)(dx + p * 8 + 4) = o1;
  }
}

__global__ void __launch_bounds__(256) k_dgamma_part(const float* dy, const uint16_t* x,
                                                     const float* r, float* P, int rows, int H) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= H) return;
  const int t0 = blockIdx.y * kGammaGroup;
  const int t1 = min(rows, t0 + kGammaGroup);
  float acc = 0.0f;
  // the loads of 16 rows are issued ahead; the sum itself stays one sequential chain
#pragma unroll 16
  for (int t = t0; t < t1; ++t)
    acc = acc + (dy[(int64_t)t * H + k] * bf16_to_f32(x[(int64_t)t * H + k])) * r[t];
  P[(int64_t)blockIdx.y * H + k] = acc;
}

__global__ void __launch_bounds__(256) k_dgamma_chain(const float* P, int nq, int H,
                                                      float* dgamma, int accumulate) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= H) return;
  float acc = accumulate ? dgamma[k] : 0.0f;
  for (int q = 0; q < nq; ++q) acc = acc + P[(int64_t)q * H + k];
  dgamma[k] = acc;
}

template <class F>
void with_bwd_modes(bool entg, bool temp, bool port, F&& f) {
  using T = std::true_type;
  using N = std::false_type;
  auto p2 = [&](auto e, auto t) {
    if (port) f(e, t, T{});
    else f(e, t, N{});
  };
  auto p1 = [&](auto e) {
    if (temp) p2(e, T{});
    else p2(e, N{});
  };
  if (entg) p1(T{});
  else p1(N{});
}

}  // namespace

hipError_t launch_rmsnorm_bwd(const RmsBwdArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_rmsnorm_bwd, dim3((unsigned)((a.rows + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dgamma(const float* dy, const uint16_t* x, const float* r, float* P, int rows,
                         int H, float* dgamma, bool accumulate, hipStream_t s) {
  const int nq = (rows + kGammaGroup - 1) / kGammaGroup;
  const unsigned cb = (unsigned)((H + 255) / 256);
  if (nq > 0) {
    hipLaunchKernelGGL(k_dgamma_part, dim3(cb, (unsigned)nq), dim3(256), 0, s, dy, x, r, P, rows,
                       H);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_dgamma_chain, dim3(cb), dim3(256), 0, s, P, nq, H, dgamma,
                     accumulate ? 1 : 0);
  return hipGetLastError();
}

// Persistent launch over batches x the A tiles x B tiles of one GEMM: one block per CU (the
// kernel's LDS allows no second), fewer when there are fewer items; the queues must be zero, and
// the kernel leaves them zero.
static bool gemm_grid(GemmArgs& q, int batches, dim3& grid) {
  const int64_t n_mt = (q.M + kGBM - 1) / kGBM, n_nt = (q.N + kGBN - 1) / kGBN;
  const int64_t n_tt = n_nt * batches;
  const int64_t items = n_mt * n_tt;
  if (items > 0x7fffffffLL - 8 * 4096) return false;
  q.n_bt = (int32_t)n_nt;
  // one band per batch: every XCD works through the batches in order, so that at any time the
  // whole device streams the same batch's A operand (one vocab segment of W for dh), as a plain
  // launch of one grid slice per batch would
  queue_setup(q, n_mt, n_tt, n_nt);
  grid = dim3((unsigned)std::min<int64_t>(items, q.n_cu > 0 ? q.n_cu : 256));
  return true;
}

hipError_t launch_gemm_dz(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (!a.queue) return hipErrorInvalidValue;
  GemmArgs q = a;
  dim3 grid;
  if (!gemm_grid(q, 1, grid)) return hipErrorInvalidConfiguration;
  with_bwd_modes(a.gH != nullptr, a.inv_tau != 1.0f, a.portable != 0,
                 [&](auto e, auto t, auto p) {
                   hipLaunchKernelGGL((k_gemm<0, e.value, t.value, p.value, false, false, false>),
                                      grid, dim3(64 * kGWaves), 0, s, q);
                 });
  return hipGetLastError();
}

hipError_t launch_gemm_out(const GemmArgs& a, int batches, bool b_trans, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0 || batches <= 0) return hipSuccess;
  if (!a.queue) return hipErrorInvalidValue;
  GemmArgs q = a;
  dim3 grid;
  if (!gemm_grid(q, batches, grid)) return hipErrorInvalidConfiguration;
  const dim3 block(64 * kGWaves);
  // dh: A (W) K-major, B (dz) K-contiguous; dW: both K-major (hidden rows, dz)
  if (b_trans) {
    if (a.accumulate) hipLaunchKernelGGL((k_gemm<1, false, false, false, true, true, true>), grid, block, 0, s, q);
    else hipLaunchKernelGGL((k_gemm<1, false, false, false, false, true, true>), grid, block, 0, s, q);
  } else {
    if (a.accumulate) hipLaunchKernelGGL((k_gemm<1, false, false, false, true, true, false>), grid, block, 0, s, q);
    else hipLaunchKernelGGL((k_gemm<1, false, false, false, false, true, false>), grid, block, 0, s, q);
  }
  return hipGetLastError();
}

hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 8192);
  hipLaunchKernelGGL(k_zero_f32, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_seg_tree(const float* part, int64_t stride, int nseg, float* out, int64_t n,
                           hipStream_t s) {
  const int64_t n4 = n / 4;
  if (n4 <= 0) return hipSuccess;
  const dim3 grid((unsigned)std::min<int64_t>((n4 + 255) / 256, 8192)), block(256);
  switch (nseg) {
    case 1: hipLaunchKernelGGL(k_seg_tree<1>, grid, block, 0, s, part, stride, out, n4); break;
    case 2: hipLaunchKernelGGL(k_seg_tree<2>, grid, block, 0, s, part, stride, out, n4); break;
    case 4: hipLaunchKernelGGL(k_seg_tree<4>, grid, block, 0, s, part, stride, out, n4); break;
    case 8: hipLaunchKernelGGL(k_seg_tree<8>, grid, block, 0, s, part, stride, out, n4); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rlk
