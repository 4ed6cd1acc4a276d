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

// Block -> (A tile, B tile), XCD-aware as in the forward: consecutive block ids go round-robin to
// the 8 XCDs, so they are remapped to let each XCD walk a contiguous range, a group of 8 A tiles
// at a time across the B tiles. Returns false for the few padding blocks.
__device__ __forceinline__ bool map_gemm(int M, int N, GTile& t) {
  const int n_mt = (M + kGBM - 1) / kGBM, n_nt = (N + kGBN - 1) / kGBN;
  const int64_t n_items = (int64_t)n_mt * n_nt;
  const int64_t nblk = (n_items + 7) / 8 * 8;
  const int64_t bid = blockIdx.x;
  if (bid >= nblk) return false;
  const int64_t L = (bid % 8) * (nblk / 8) + bid / 8;
  if (L >= n_items) return false;
  constexpr int GV = 8;
  const int64_t grp = L / ((int64_t)GV * n_nt);
  const int first = (int)(grp * GV);
  const int gsz = min(GV, n_mt - first);
  const int64_t within = L - grp * GV * n_nt;
  const int mt = first + (int)(within % gsz);
  const int nt = (int)(within / gsz);
  t.m0 = uni(mt * kGBM);
  t.mrows = uni(min(kGBM, M - mt * kGBM));
  t.n0 = uni(nt * kGBN);
  t.nrows = uni(min(kGBN, N - nt * kGBN));
  return true;
}

int64_t gemm_blocks(int M, int N) {
  const int64_t n = (int64_t)((M + kGBM - 1) / kGBM) * ((N + kGBN - 1) / kGBN);
  return (n + 7) / 8 * 8;
}

// Output row of this lane's B row in B block j of the wave (OUT epilogue), or null for a row past
// the tile or a padding row of the segment-padded vocab layout. 32-bit index math: B rows are
// below 2^31.
__device__ __forceinline__ const float* out_row(const GemmArgs& a, const float* C, const GTile& t,
                                                int wt, int j, int lane) {
  const int nn = 16 * (wt * kGNB16 + j) + (lane & 15);
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

// One B1 value.
template <bool ENTG, bool TEMP, bool PORT>
__device__ __forceinline__ uint16_t dz_one(float acc, int v, int y, float g, float l, float gh,
                                           float e, float inv_tau) {
  const float zp = TEMP ? acc * inv_tau : acc;
  const float p = EXP<PORT>(zp - l);
  const float d = (v == y) ? 1.0f - p : -p;
  float q = g * d;
  if constexpr (ENTG) q = q - gh * (p * ((zp - l) + e));
  if constexpr (TEMP) q = q * inv_tau;
  // bf16_rne (NaN kept quiet) and the padded-row zero as mask arithmetic: the compiler would
  // otherwise wrap each element in branches
  const uint32_t u = __float_as_uint(q);
  const uint32_t rne = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const uint32_t nan = 0u - (uint32_t)((u & 0x7fffffffu) > 0x7f800000u);
  const uint32_t bits = (rne & ~nan) | (((u >> 16) | 0x40u) & nan);
  return (uint16_t)(bits & (0u - (uint32_t)(y >= 0)));
}

// The backward's NT GEMM tile kernel (see GemmArgs). EPI 0 = DZ, 1 = OUT.
template <int EPI, bool ENTG, bool TEMP, bool PORT, bool ACC, bool ATR, bool BTR>
__global__ void __launch_bounds__(64 * kGWaves) k_gemm(const GemmArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds_a0[kGBM * kRowBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_a1[kGBM * kRowBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_b0[kGBN * kRowBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_b1[kGBN * kRowBytes];

  GTile t;
  if (!map_gemm(a.M, a.N, t)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wv = wave % kGVW;
  const int wt = wave / kGVW;
  const int64_t yb = blockIdx.y;
  const uint16_t* __restrict__ Bt =
      BTR ? a.B + yb * a.b_batch + t.n0 : a.B + yb * a.b_batch + (int64_t)t.n0 * a.ldb;

  // Staging offsets as in the forward: rows past the tile are clamped to its last row. DZ runs
  // over the segment-padded vocab positions: tile row m reads W row v(m), a padding position
  // the last row of its segment (its result is replaced by 0). v(m) never decreases, and the
  // tile's real rows are consecutive in W, so one descriptor from v(first) covers them.
  uint32_t ago[kGWI], bgo[kGHI];
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
  const __amdgpu_buffer_rsrc_t ra =
      ATR ? make_rsrc(At, tr_bytes(a.ka_rows, a.lda, t.m0))
          : make_rsrc(At, (int)(((a_rows - 1) * a.lda + a.K) * 2));
  const __amdgpu_buffer_rsrc_t rb =
      BTR ? make_rsrc(Bt, tr_bytes(a.kb_rows, a.ldb, t.n0))
          : make_rsrc(Bt, (int)(((int64_t)(t.nrows - 1) * a.ldb + a.K) * 2));

  float* __restrict__ C = EPI == 1 ? a.C + yb * a.c_batch : nullptr;
  f32x4 acc[kGVB16][kGNB16];
#pragma unroll
  for (int i = 0; i < kGVB16; ++i)
#pragma unroll
    for (int j = 0; j < kGNB16; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.0f;
  if constexpr (EPI == 1 && ACC) {
    static_for<kGNB16>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const float* crow = out_row(a, C, t, wt, j, lane);
      if (!crow) return;
      const int mb = t.m0 + 16 * wv * kGVB16 + 4 * (lane >> 4);
      static_for<kGVB16>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        if (mb + 16 * i < a.M) acc[i][j] = *(const f32x4*)(crow + mb + 16 * i);
      });
    });
  }
  nt_mainloop<kGWaves, kGVB16, kGNB16, kGWI, kGHI, ATR, BTR>(
      acc, lds_a0, lds_a1, lds_b0, lds_b1, ra, rb, ago, bgo, a.K / kKStage, wave, lane, wv, wt,
      (uint32_t)(64 * a.lda * 2), (uint32_t)(64 * a.ldb * 2));

  // The epilogues index the accumulators with compile-time constants (static_for): a runtime
  // index would move them to scratch. The lane id goes through an empty asm so that the compiler
  // recomputes every address from it instead of keeping the prologue's alive across the K loop.
  int ln = lane;
  __asm__ volatile("" : "+v"(ln));
  if constexpr (EPI == 1) {
    // one output row pointer per B block (row(n) needs one division), then constant offsets
    static_for<kGNB16>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      float* crow = const_cast<float*>(out_row(a, C, t, wt, j, ln));
      if (!crow) return;
      const int mb = t.m0 + 16 * wv * kGVB16 + 4 * (ln >> 4);
      static_for<kGVB16>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        if (mb + 16 * i < a.M) *(f32x4*)(crow + mb + 16 * i) = acc[i][j];
      });
    });
  } else {
    // B1 on the result registers: lane holds rows n = token (lane & 15 of each B block) and
    // 4 consecutive vocab indices m per A block
    int yj[kGNB16];
    float gj[kGNB16], lj[kGNB16], hj[kGNB16], ej[kGNB16];
#pragma unroll
    for (int j = 0; j < kGNB16; ++j) {
      const int nn = 16 * (wt * kGNB16 + j) + (ln & 15);
      const bool ok = nn < t.nrows;
      const int64_t n = t.n0 + (ok ? nn : 0);
      yj[j] = ok ? a.targets[n] : -1;
      gj[j] = a.g[n];
      lj[j] = a.lse[n];
      hj[j] = ENTG ? a.gH[n] : 0.0f;
      ej[j] = ENTG ? a.ent[n] : 0.0f;
    }
    // hoisted addressing: the lane's dz row for B block 0 (block j adds 16 rows); positions,
    // segments and vocab indices in 32-bit math (< 2^31)
    const int64_t tl = t.n0 + 16 * wt * kGNB16 + (ln & 15);
    uint16_t* const dzr = a.dz + tl * a.lddz;
    const int64_t dz_j = 16 * a.lddz;
    const uint32_t L = (uint32_t)a.seg_len, Lp = (uint32_t)a.seg_pad;
    const uint32_t cb = (uint32_t)(t.m0 + 16 * wv * kGVB16 + 4 * (ln >> 4));
    static_for<kGVB16>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      // 4 consecutive padded positions col0 .. col0+3 (one segment: Lp is a multiple of 128)
      const uint32_t col0 = cb + 16 * i;
      const uint32_t sg = col0 / Lp;
      const uint32_t c0 = col0 - sg * Lp;  // position inside the segment
      const int v0 = (int)(a.v_base + sg * L + c0);  // vocab index of col0 when c0 < L
      const bool col_ok = (int)col0 < a.M;
      static_for<kGNB16>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        const int nn = 16 * (wt * kGNB16 + j) + (ln & 15);
        if (nn >= t.nrows || !col_ok) return;
        uint16_t b[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint16_t x = dz_one<ENTG, TEMP, PORT>(acc[i][j][r], v0 + r, yj[j], gj[j], lj[j],
                                                      hj[j], ej[j], a.inv_tau);
          b[r] = c0 + r < L ? x : (uint16_t)0;
        }
        const uint32_t w0 = (uint32_t)b[0] | ((uint32_t)b[1] << 16);
        const uint32_t w1 = (uint32_t)b[2] | ((uint32_t)b[3] << 16);
        *(uint2*)(dzr + j * dz_j + col0) = make_uint2(w0, w1);
      });
    });
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

hipError_t launch_gemm_dz(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  const int64_t blocks = gemm_blocks(a.M, a.N);
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  with_bwd_modes(a.gH != nullptr, a.inv_tau != 1.0f, a.portable != 0,
                 [&](auto e, auto t, auto p) {
                   hipLaunchKernelGGL((k_gemm<0, e.value, t.value, p.value, false, false, false>),
                                      dim3((unsigned)blocks), dim3(64 * kGWaves), 0, s, a);
                 });
  return hipGetLastError();
}

hipError_t launch_gemm_out(const GemmArgs& a, int batches, bool b_trans, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0 || batches <= 0) return hipSuccess;
  const int64_t blocks = gemm_blocks(a.M, a.N);
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks, (unsigned)batches), block(64 * kGWaves);
  // dh: A (W) K-major, B (dz) K-contiguous; dW: both K-major (hidden rows, dz)
  if (b_trans) {
    if (a.accumulate) hipLaunchKernelGGL((k_gemm<1, false, false, false, true, true, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_gemm<1, false, false, false, false, true, true>), grid, block, 0, s, a);
  } else {
    if (a.accumulate) hipLaunchKernelGGL((k_gemm<1, false, false, false, true, true, false>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_gemm<1, false, false, false, false, true, false>), grid, block, 0, s, a);
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
