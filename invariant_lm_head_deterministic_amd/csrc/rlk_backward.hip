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
// Layout of the backward's intermediates (all in the caller's workspace): dz [rows][S_c Lp] and
// dzt [S_c Lp][rows padded] hold vocab index v = s L + c at the segment-padded position s Lp + c
// (L = V / S_c, Lp = L rounded up to 128); WT [H][S_c Lp] and hT [H][rows padded] are the
// transposed operands, so every GEMM here is an NT GEMM with K contiguous in both operands, the
// shape of the forward's K loop (nt_mainloop).

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

// segment-padded position of vocab index v, and back (-1 for a padding position)
__device__ __forceinline__ int64_t pad_col(int64_t v, int64_t L, int64_t Lp) {
  const int64_t s = v / L;
  return v + s * (Lp - L);
}
__device__ __forceinline__ int64_t unpad_row(int64_t n, int64_t L, int64_t Lp) {
  const int64_t s = n / Lp;
  const int64_t c = n - s * Lp;
  return c < L ? s * L + c : -1;
}

// One B1 value.
template <bool ENTG, bool TEMP, bool PORT>
__device__ __forceinline__ uint16_t dz_one(float acc, int64_t v, int y, float g, float l, float gh,
                                           float e, float inv_tau) {
  if (y < 0) return 0;
  const float zp = TEMP ? acc * inv_tau : acc;
  const float p = EXP<PORT>(zp - l);
  const float d = (v == (int64_t)y) ? 1.0f - p : -p;
  float q = g * d;
  if constexpr (ENTG) q = q - gh * (p * ((zp - l) + e));
  if constexpr (TEMP) q = q * inv_tau;
  return bf16_rne(q);
}

// The backward's NT GEMM tile kernel (see GemmArgs). EPI 0 = DZ, 1 = OUT.
template <int EPI, bool ENTG, bool TEMP, bool PORT, bool ACC>
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
  const uint16_t* __restrict__ At = a.A + yb * a.a_batch + (int64_t)t.m0 * a.lda;
  const uint16_t* __restrict__ Bt = a.B + yb * a.b_batch + (int64_t)t.n0 * a.ldb;

  // staging offsets as in the forward: rows past the tile are clamped to its last row
  uint32_t ago[kGWI], bgo[kGHI];
#pragma unroll
  for (int q = 0; q < kGWI; ++q) {
    const int r = 8 * (q * kGWaves + wave) + (lane >> 3);
    const int c = (lane & 7) ^ swz(r);
    ago[q] = (uint32_t)(((int64_t)min(r, t.mrows - 1) * a.lda + c * 8) * 2);
  }
#pragma unroll
  for (int q = 0; q < kGHI; ++q) {
    const int r = 8 * (q * kGWaves + wave) + (lane >> 3);
    const int c = (lane & 7) ^ swz(r);
    bgo[q] = (uint32_t)(((int64_t)min(r, t.nrows - 1) * a.ldb + c * 8) * 2);
  }
  const __amdgpu_buffer_rsrc_t ra =
      make_rsrc(At, (int)(((int64_t)(t.mrows - 1) * a.lda + a.K) * 2));
  const __amdgpu_buffer_rsrc_t rb =
      make_rsrc(Bt, (int)(((int64_t)(t.nrows - 1) * a.ldb + a.K) * 2));

  float* __restrict__ C = EPI == 1 ? a.C + yb * a.c_batch : nullptr;
  f32x4 acc[kGVB16][kGNB16];
#pragma unroll
  for (int i = 0; i < kGVB16; ++i)
#pragma unroll
    for (int j = 0; j < kGNB16; ++j) {
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.0f;
      if constexpr (EPI == 1 && ACC) {
        const int m = t.m0 + 16 * (wv * kGVB16 + i) + 4 * (lane >> 4);
        const int nn = 16 * (wt * kGNB16 + j) + (lane & 15);
        const int64_t n = t.n0 + nn;
        const int64_t row = a.map_rows ? unpad_row(n, a.seg_len, a.seg_pad) : n;
        if (nn < t.nrows && m < a.M && row >= 0) acc[i][j] = *(const f32x4*)(C + row * a.ldc + m);
      }
    }
  nt_mainloop<kGWaves, kGVB16, kGNB16, kGWI, kGHI>(acc, lds_a0, lds_a1, lds_b0, lds_b1, ra, rb,
                                                   ago, bgo, a.K / kKStage, wave, lane, wv, wt);

  // The epilogues index the accumulators with compile-time constants (static_for): a runtime
  // index would move them to scratch. The lane id is read afresh (mbcnt) so that no index value
  // computed before the K loop stays live across it.
  const int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  if constexpr (EPI == 1) {
    static_for<kGVB16>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      static_for<kGNB16>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        const int m = t.m0 + 16 * (wv * kGVB16 + i) + 4 * (ln >> 4);
        const int nn = 16 * (wt * kGNB16 + j) + (ln & 15);
        const int64_t n = t.n0 + nn;
        const int64_t row = a.map_rows ? unpad_row(n, a.seg_len, a.seg_pad) : n;
        if (nn < t.nrows && m < a.M && row >= 0) *(f32x4*)(C + row * a.ldc + m) = acc[i][j];
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
    const bool fast = (a.seg_len & 3) == 0;
    static_for<kGVB16>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const int64_t v0 = t.m0 + 16 * (wv * kGVB16 + i) + 4 * (ln >> 4);
      if (v0 >= a.V) return;
      const int64_t s0 = v0 / a.seg_len;
      const int64_t col0 = v0 + s0 * (a.seg_pad - a.seg_len);
      static_for<kGNB16>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        const int nn = 16 * (wt * kGNB16 + j) + (ln & 15);
        if (nn >= t.nrows) return;
        const int64_t n = t.n0 + nn;
        uint16_t b[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          b[r] = dz_one<ENTG, TEMP, PORT>(acc[i][j][r], v0 + r, yj[j], gj[j], lj[j], hj[j], ej[j],
                                          a.inv_tau);
        if (fast && v0 + 3 < a.V) {
          // the 4 indices share a segment: contiguous, 8-byte aligned positions
          if (a.dz) {
            const uint32_t lo = (uint32_t)b[0] | ((uint32_t)b[1] << 16);
            const uint32_t hi = (uint32_t)b[2] | ((uint32_t)b[3] << 16);
            *(uint2*)(a.dz + n * a.lddz + col0) = make_uint2(lo, hi);
          }
          if (a.dzt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) a.dzt[(col0 + r) * a.lddzt + n] = b[r];
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int64_t v = v0 + r;
            if (v >= a.V) continue;
            const int64_t col = pad_col(v, a.seg_len, a.seg_pad);
            if (a.dz) a.dz[n * a.lddz + col] = b[r];
            if (a.dzt) a.dzt[col * a.lddzt + n] = b[r];
          }
        }
      });
    });
  }
}

// 64 x 64 transpose tile through LDS (see TransposeArgs). The tile is stored as [c][j] so that
// the output rows leave LDS as 16-byte vectors and 8 lanes write 128 contiguous bytes.
__global__ void __launch_bounds__(256) k_transpose(const TransposeArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64][72];
  const int64_t j0 = (int64_t)blockIdx.x * 64;
  const int64_t c0 = (int64_t)blockIdx.y * 64;
  for (int q = threadIdx.x; q < 64 * 8; q += 256) {
    const int jj = q >> 3, pc = q & 7;
    const int64_t j = j0 + jj;
    const int64_t s = j / a.Lp, cc = j - s * a.Lp;
    const int64_t r = s * a.L + cc;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (j < a.J && cc < a.L && r < a.R) v = *(const u32x4*)(a.in + r * a.ldi + c0 + pc * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[pc * 8 + 2 * e][jj] = (uint16_t)(v[e] & 0xffffu);
      tile[pc * 8 + 2 * e + 1][jj] = (uint16_t)(v[e] >> 16);
    }
  }
  __syncthreads();
  for (int q = threadIdx.x; q < 64 * 8; q += 256) {
    const int cr = q >> 3, pj = q & 7;
    const int64_t j = j0 + pj * 8;
    if (j >= a.J) continue;
    *(u32x4*)(a.out + (c0 + cr) * a.ldo + j) = *(const u32x4*)(&tile[cr][pj * 8]);
  }
}

__global__ void k_zero_rect(uint16_t* p, int64_t ld, int64_t r0, int64_t r1, int64_t c0,
                            int64_t c1) {
  const int64_t w = c1 - c0;
  const int64_t n = (r1 - r0) * w;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = r0 + i / w, c = c0 + i % w;
    p[r * ld + c] = 0;
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
                   hipLaunchKernelGGL((k_gemm<0, e.value, t.value, p.value, false>),
                                      dim3((unsigned)blocks), dim3(64 * kGWaves), 0, s, a);
                 });
  return hipGetLastError();
}

hipError_t launch_gemm_out(const GemmArgs& a, int batches, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0 || batches <= 0) return hipSuccess;
  const int64_t blocks = gemm_blocks(a.M, a.N);
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks, (unsigned)batches);
  if (a.accumulate)
    hipLaunchKernelGGL((k_gemm<1, false, false, false, true>), grid, dim3(64 * kGWaves), 0, s, a);
  else
    hipLaunchKernelGGL((k_gemm<1, false, false, false, false>), grid, dim3(64 * kGWaves), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_transpose(const TransposeArgs& a, hipStream_t s) {
  if (a.J <= 0 || a.C <= 0) return hipSuccess;
  const dim3 grid((unsigned)((a.J + 63) / 64), (unsigned)((a.C + 63) / 64));
  hipLaunchKernelGGL(k_transpose, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_zero_rect(uint16_t* p, int64_t ld, int64_t r0, int64_t r1, int64_t c0,
                            int64_t c1, hipStream_t s) {
  const int64_t n = (r1 - r0) * (c1 - c0);
  if (n <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(k_zero_rect, dim3((unsigned)blocks), dim3(256), 0, s, p, ld, r0, r1, c0, c1);
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
