// Device-side building blocks shared by the forward (rlk_kernels.hip) and backward
// (rlk_backward.hip) kernels: the contract's primitives, bf16 conversions, buffer descriptors and
// direct-to-LDS copies, and the staged MFMA K loop of a 256 x 256-style NT tile.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "rlk_internal.h"

namespace rlk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 0x1.715476p+0f;  // fl32(log2(e))
constexpr float kLn2 = 0x1.62e430p-1f;    // fl32(ln(2))
constexpr int kRowBytes = kKStage * 2;    // bytes of one staged row (128)

__device__ __forceinline__ float c_exp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
__device__ __forceinline__ float c_log(float x) { return __builtin_amdgcn_logf(x) * kLn2; }
__device__ __forceinline__ float c_rsq(float x) { return __builtin_amdgcn_rsqf(x); }

// Portable EXP and LOG (RLK_FLAG_PORTABLE_EXP, C11p): every step is one IEEE fp32 operation
// rounded to nearest even, a round-to-integral-even, or an exact integer or bit operation, so
// any IEEE machine that runs the same steps gets the same bits.
//  EXP: x = n ln2 + r by Cody and Waite's reduction, ln2 = C1 + C2 with C1 = 0.693359375 (9
//  significant bits, so n C1 is exact); e^r by its Taylor polynomial to r^7/7! in Horner form
//  (|r| <= 0.347: truncation below 6e-9 relative); then the scaling by 2^n, built from exponent
//  bits, in two steps near overflow and below 2^-126 so that every result rounds once.
//  LOG: x = (1 + f) 2^k with 1 + f in [sqrt(1/2), sqrt(2)]; s = f / (2 + f) and
//  log(1 + f) = 2 atanh(s) by its odd series to s^11/11 (|s| <= 0.172: truncation below 6e-11),
//  arranged around the exact f; then k C1 + (that + k C2). RSQ is 1 / sqrt(x), both correctly
//  rounded. Measured against float64: EXP within 1.2 ulp, LOG 0.83 ulp, RSQ 1.5 ulp.
constexpr float kLn2C1 = 0x1.63p-1f;        // 0.693359375
constexpr float kLn2C2 = -0x1.bd0106p-13f;  // fl32(ln2 - C1)

__device__ __forceinline__ float pow2i(int n) { return __int_as_float((n + 127) << 23); }

__device__ __forceinline__ float p_exp(float x) {
  // Branch-free: out-of-range inputs are clamped for the arithmetic and their result replaced.
  const float xc = fminf(fmaxf(x, -0x1.9fe368p+6f), 0x1.62e430p+6f);
  const float nf = __builtin_rintf(xc * kLog2e);
  const int n = (int)nf;  // -150 .. 128
  const float r = (xc - nf * kLn2C1) - nf * kLn2C2;
  float p = 0x1.a01a02p-13f;    // 1/7!
  p = p * r + 0x1.6c16c2p-10f;  // 1/6!
  p = p * r + 0x1.111112p-7f;   // 1/5!
  p = p * r + 0x1.555556p-5f;   // 1/4!
  p = p * r + 0x1.555556p-3f;   // 1/3!
  p = p * r + 0.5f;
  p = p * r + 1.0f;
  p = p * r + 1.0f;
  // 2^n as 2^(n - n2) 2^n2 with both factors normal: the first product is exact, the second
  // rounds once (n2 = 0 in the normal range, -64 below 2^-126, +1 at n = 128).
  const int n2 = n < -126 ? -64 : (n > 127 ? 1 : 0);
  float y = (p * pow2i(n - n2)) * pow2i(n2);
  y = x < -0x1.9fe368p+6f ? 0.0f : y;        // below fl32(ln(2^-150)): rounds to +0
  y = x > 0x1.62e430p+6f ? INFINITY : y;     // above fl32(ln(FLT_MAX)): overflows
  return x != x ? x : y;
}

__device__ __forceinline__ float p_log(float x) {
  if (x != x || x < 0.0f) return __builtin_nanf("");
  if (x == 0.0f) return -INFINITY;
  if (x == INFINITY) return x;
  int adj = 0;
  if (x < 0x1p-126f) {
    x = x * 0x1p23f;  // exact: subnormal -> normal
    adj = -23;
  }
  const uint32_t u = __float_as_uint(x);
  int k = (int)((u >> 23) & 0xffu) - 127 + adj;
  float m = __uint_as_float((u & 0x007fffffu) | 0x3f800000u);  // [1, 2)
  if (m > 0x1.6a09e6p+0f) {  // fl32(sqrt(2))
    m = m * 0.5f;
    k = k + 1;
  }
  const float f = m - 1.0f;
  const float s = f / (f + 2.0f);
  const float z = s * s;
  float R = 0x1.745d18p-3f;    // 2/11
  R = R * z + 0x1.c71c72p-3f;  // 2/9
  R = R * z + 0x1.24924ap-2f;  // 2/7
  R = R * z + 0x1.99999ap-2f;  // 2/5
  R = R * z + 0x1.555556p-1f;  // 2/3
  R = R * z;
  const float hfsq = 0.5f * (f * f);
  const float kf = (float)k;
  // log(1 + f) = 2s + s R = f - (f^2/2 - s (f^2/2 + R)): the exact f carries the leading bits
  return kf * kLn2C1 + (f - (hfsq - (s * (hfsq + R) + kf * kLn2C2)));
}

__device__ __forceinline__ float p_rsq(float x) { return 1.0f / __builtin_sqrtf(x); }

template <bool PORT>
__device__ __forceinline__ float EXP(float x) {
  if constexpr (PORT) return p_exp(x);
  else return c_exp(x);
}
template <bool PORT>
__device__ __forceinline__ float LOG(float x) {
  if constexpr (PORT) return p_log(x);
  else return c_log(x);
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Staged tiles hold rows of 128 bytes (64 bf16 of K) as 8 pieces of 16 bytes. Piece c of row r
// sits at position c ^ ((r >> 1) & 7): a fragment read of 16 consecutive rows (one pass of a
// 16-byte-per-lane LDS read over 64 banks) then touches every bank exactly once.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

typedef __attribute__((address_space(3))) void* lptr_t;

// Buffer descriptor over `bytes` bytes from `base` (raw, unstrided; the word-3 value selects
// 32-bit data format, which makes the descriptor valid for untyped loads).
// The descriptor must live in SGPRs: its inputs go through readfirstlane (they are uniform by
// construction) so that the compiler never wraps a DMA in a loop over lanes.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  const uint64_t b = (uint64_t)base;
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)b);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)(b >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void*)((hi << 32) | lo), (short)0,
                                           __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uni64(int64_t x) {
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)x);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)((uint64_t)x >> 32));
  return (int64_t)((hi << 32) | lo);
}

// Asynchronous 16-byte-per-lane copy global -> LDS (buffer_load_dwordx4 ... lds): lane l's bytes
// come from byte offset voff + soff of the descriptor and land at lds_base + 16 l.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds_base, uint32_t voff,
                                      uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lptr_t)lds_base, 16, voff, soff, 0, 0);
}

__device__ __forceinline__ void wait_dma() { __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Balanced pairwise sum of N = 2^k values in index order (the C5/C9 tree).
template <int N>
__device__ __forceinline__ float tree_sum(const float* v) {
  if constexpr (N == 1) {
    return v[0];
  } else {
    float w[N / 2];
#pragma unroll
    for (int i = 0; i < N / 2; ++i) w[i] = v[2 * i] + v[2 * i + 1];
    return tree_sum<N / 2>(w);
  }
}

// ---------------------------------------------------------------------------------------------
// The staged K loop of an NT tile: acc[i][j] += A-rows x B-rows^T over nk stages of 64 K, both
// operands bf16 with K contiguous, fp32 accumulation in one v_mfma_f32_16x16x32_bf16 chain per
// result element with K ascending 32 at a time (C1). A rows are the MFMA rows: the result block
// gives lane l the A rows 4 (l >> 4) + r (r = register) and the B row l & 15. A wave owns VB16
// A blocks of 16 (from A row 16 wv VB16) and NB16 B blocks of 16 (from B row 16 wt NB16) of the
// block's staged tile.
//
// Staging: direct-to-LDS DMA. Instruction q of this wave fills the 8 staged rows from
// 8 (q NWAVES + wave); ago / bgo are the per-lane byte offsets of those rows' pieces at K stage
// 0 (the caller clamps rows past its tile, swizzles the piece and applies the row stride); the K
// stage is the scalar offset. nk must be even and >= 2.
//
// Two LDS buffers per operand, distinct objects, so that a DMA into one never makes the compiler
// wait before reads of the other. Stage k: sub-step 0 runs from the fragments in registers while
// reading sub-step 1's; then this wave's DMA of stage k+1 is waited and all waves meet (stage k+1
// has landed everywhere, and every read of stage k's buffer is done); sub-step 1 then issues the
// DMA of stage k+2 into stage k's buffer and reads the first fragments of stage k+1. The last two
// stages issue no DMA and their final fragment reads are unused (in bounds).
// K-major ("transposed") staging of an operand, for operands stored with K as the row index
// (the backward's W, hidden rows and dz): a stage holds 64 K rows of the block's 256 M (or N)
// indices, 512 bytes per row, and piece p (8 indices) of row r sits at slot p ^ tswz(r). A
// fragment is read with two ds_read_b64_tr_b16 (gfx950's transposing LDS load: within each 16
// lanes, source lane 4k + q supplies 4 consecutive values and lane i receives value i % 4 of
// source 4k + i / 4, k = 0..3 - pinned by a probe): source lane j of lane group g reads row
// 8g + j / 4 (and 4 rows further for the second read) at the 4 indices from 4 (j % 4), so lane
// i of group g receives K rows 8g .. 8g+7 of index i: the MFMA operand layout. The 16 rows one
// read touches (4 per group, groups 8 rows apart) take 8 swizzle values twice each, the 2-way
// minimum of a 512-byte read over 64 banks.
constexpr int kTRowBytes = 512;
__device__ __forceinline__ int tswz(int r) { return 2 * ((r & 3) | ((r >> 1) & 4)); }

__device__ __forceinline__ bf16x8 tr_read(const uint8_t* tile, int off) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef short v8s __attribute__((ext_vector_type(8)));
  typedef __attribute__((address_space(3))) v4s* lv4s;
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lv4s)(tile + off));
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lv4s)(tile + off + 4 * kTRowBytes));
  const v8s c = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

// Per-lane byte offset (sub-step 0, block 0) and block XOR of transposed fragment reads: block
// b of sub-step s is read at base + 16384 s + ((32 b) ^ x).
__device__ __forceinline__ void tr_lane(int lane, int& base, int& x) {
  const int j = lane & 15, g = lane >> 4;
  const int row = 8 * g + (j >> 2);
  base = row * kTRowBytes + 16 * ((j & 3) >> 1) + 8 * (j & 1);
  x = 16 * tswz(row);
}

// One K stage of two K-contiguous operands, staged as rows of kRowBytes: DMA instruction q of
// this wave fills the 8 staged rows from 8 (q NWAVES + wave); kc is the stage.
template <int NWAVES, int WI, int HI>
__device__ __forceinline__ void issue_stage(__amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t rh,
                                            const uint32_t (&wgo)[WI], const uint32_t (&hgo)[HI],
                                            int kc, uint8_t* lw, uint8_t* lh, int wave) {
  const uint32_t so = (uint32_t)kc * kRowBytes;
#pragma unroll
  for (int q = 0; q < WI; ++q) dma16(rw, lw + 8 * (q * NWAVES + wave) * kRowBytes, wgo[q], so);
#pragma unroll
  for (int q = 0; q < HI; ++q) dma16(rh, lh + 8 * (q * NWAVES + wave) * kRowBytes, hgo[q], so);
}

struct NoHook {
  __device__ __forceinline__ void operator()() const {}
};

// The K loop of one output tile. PRE: the caller has already issued stages 0 and 1 into
// (lds_w0, lds_h0) and (lds_w1, lds_h1) and every vector memory operation this wave issued
// since then may be waited for (the loop starts with vmcnt(0)). hook() runs once, after the
// barrier that publishes stage 0, before any fragment read.
template <int NWAVES, int VB16, int NB16, int WI, int HI, bool ATR, bool BTR, bool PRE, class Hook>
__device__ __forceinline__ void nt_mainloop_x(f32x4 (&acc)[VB16][NB16], uint8_t* lds_w0,
                                              uint8_t* lds_w1, uint8_t* lds_h0, uint8_t* lds_h1,
                                              __amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t rh,
                                              const uint32_t (&wgo)[WI], const uint32_t (&hgo)[HI],
                                              int nk, int wave, int lane, int wv, int wt,
                                              uint32_t sa, uint32_t sb, Hook& hook) {
  // sa / sb: bytes from one K stage to the next of a transposed operand (64 rows)
  auto issue = [&](int kc, uint8_t* lw, uint8_t* lh) {
    const uint32_t so = (uint32_t)kc * kRowBytes;
    const uint32_t soa = ATR ? (uint32_t)kc * sa : so;
    const uint32_t sob = BTR ? (uint32_t)kc * sb : so;
#pragma unroll
    for (int q = 0; q < WI; ++q) dma16(rw, lw + 8 * (q * NWAVES + wave) * kRowBytes, wgo[q], soa);
#pragma unroll
    for (int q = 0; q < HI; ++q) dma16(rh, lh + 8 * (q * NWAVES + wave) * kRowBytes, hgo[q], sob);
  };
  int tbase = 0, tx = 0;
  if constexpr (ATR || BTR) tr_lane(lane, tbase, tx);
  auto fragA = [&](const uint8_t* lw, int ns, int i) -> bf16x8 {
    if constexpr (ATR) return tr_read(lw, 16384 * ns + tbase + ((32 * (wv * VB16 + i)) ^ tx));
    else return *(const bf16x8*)(lw + 16 * wv * VB16 * kRowBytes + i * 16 * kRowBytes +
                                 (lane & 15) * kRowBytes +
                                 (((4 * ns + (lane >> 4)) ^ swz(lane & 15)) << 4));
  };
  auto fragB = [&](const uint8_t* lh, int ns, int j) -> bf16x8 {
    if constexpr (BTR) return tr_read(lh, 16384 * ns + tbase + ((32 * (wt * NB16 + j)) ^ tx));
    else return *(const bf16x8*)(lh + 16 * wt * NB16 * kRowBytes + j * 16 * kRowBytes +
                                 (lane & 15) * kRowBytes +
                                 (((4 * ns + (lane >> 4)) ^ swz(lane & 15)) << 4));
  };

  // Fragment reads: sub-step s (K 32s .. 32s+31 of a stage) reads piece 4s + (lane >> 4) of row
  // lane & 15 of each 16-row block; every block row has the same (row >> 1) & 7 as lane & 15,
  // so one lane offset per sub-step serves all blocks, at constant 2 KB strides.
  const int r16 = lane & 15;
  int loff[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) loff[s] = r16 * kRowBytes + (((4 * s + (lane >> 4)) ^ swz(r16)) << 4);
  const int a0 = 16 * wv * VB16 * kRowBytes, b0 = 16 * wt * NB16 * kRowBytes;
  // Register budget (2 waves per SIMD): the A fragments are single-buffered, each re-read right
  // after the MFMAs of its row block (its next use is (VB16-1) NB16 MFMAs later); the B
  // fragments, used by every row block, are double-buffered.
  bf16x8 fa[VB16], fb[2][NB16];
  // One sub-step: MFMAs on fa / fb[cb] while reading the fragments of sub-step ns of the
  // buffers (lw, lh) into fa / fb[1-cb]; ND DMA instructions spread over the MFMAs.
  constexpr int NM = VB16 * NB16;  // MFMAs per sub-step
  auto sub = [&](auto cb_c, auto nd_c, const uint8_t* lw, const uint8_t* lh, int ns) {
    constexpr int cb = decltype(cb_c)::value;
    constexpr int ND = decltype(nd_c)::value;
    const uint8_t* pa = lw + a0 + loff[ns];
    const uint8_t* pb = lh + b0 + loff[ns];
#pragma unroll
    for (int j = 0; j < NB16; ++j) {
      if constexpr (BTR) fb[1 - cb][j] = fragB(lh, ns, j);
      else fb[1 - cb][j] = *(const bf16x8*)(pb + j * 16 * kRowBytes);
    }
#pragma unroll
    for (int i = 0; i < VB16; ++i) {
#pragma unroll
      for (int j = 0; j < NB16; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[cb][j], acc[i][j], 0, 0, 0);
      if constexpr (ATR) fa[i] = fragA(lw, ns, i);
      else fa[i] = *(const bf16x8*)(pa + i * 16 * kRowBytes);
    }
    // order: the B reads interleaved with the first row block's MFMAs, then one A read after
    // each row block; DMA instructions every EV MFMAs
    constexpr int NDs = ND > 0 ? ND : 1;
    constexpr int EV = ND > 0 ? (NM / NDs > 0 ? NM / NDs : 1) : NM + 1;
    constexpr int INLOOP = ND > 0 ? (NM / EV < ND ? NM / EV : ND) : 0;
#pragma unroll
    for (int n = 0; n < NM; ++n) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (n < NB16) __builtin_amdgcn_sched_group_barrier(0x100, BTR ? 2 : 1, 0);
      if (n % NB16 == NB16 - 1) __builtin_amdgcn_sched_group_barrier(0x100, ATR ? 2 : 1, 0);
      if (ND > 0 && n % EV == EV - 1 && n / EV < INLOOP)
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    if constexpr (ND > INLOOP) __builtin_amdgcn_sched_group_barrier(0x020, ND - INLOOP, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using CD = std::integral_constant<int, WI + HI>;

  auto stage = [&](auto dma, int k, uint8_t* cw, uint8_t* ch, const uint8_t* nw,
                   const uint8_t* nh) {
    constexpr bool D = decltype(dma)::value;
    sub(C0{}, C0{}, cw, ch, 1);
    wait_dma();
    __syncthreads();
    if constexpr (D) {
      issue(k + 2, cw, ch);
      sub(C1{}, CD{}, nw, nh, 0);
    } else {
      sub(C1{}, C0{}, nw, nh, 0);
    }
  };
  if constexpr (PRE) {
    wait_dma();
  } else {
    issue(0, lds_w0, lds_h0);
    issue(nk > 1 ? 1 : 0, lds_w1, lds_h1);
    __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(WI + HI) : "memory");
  }
  __syncthreads();
  hook();
  {
    const uint8_t* pa = lds_w0 + a0 + loff[0];
    const uint8_t* pb = lds_h0 + b0 + loff[0];
#pragma unroll
    for (int j = 0; j < NB16; ++j) {
      if constexpr (BTR) fb[0][j] = fragB(lds_h0, 0, j);
      else fb[0][j] = *(const bf16x8*)(pb + j * 16 * kRowBytes);
    }
#pragma unroll
    for (int i = 0; i < VB16; ++i) {
      if constexpr (ATR) fa[i] = fragA(lds_w0, 0, i);
      else fa[i] = *(const bf16x8*)(pa + i * 16 * kRowBytes);
    }
  }
  // nothing scalar left in flight when the loop starts: a pending scalar load there makes every
  // iteration wait for all LDS reads (lgkmcnt(0)) instead of only the oldest fragments. The
  // builtin (s_waitcnt lgkmcnt(0), vmcnt and expcnt unconstrained) is visible to the compiler's
  // wait-insertion pass; an inline-asm wait would not be.
  __builtin_amdgcn_s_waitcnt(0xC07F);
  int k = 0;
  for (; k + 2 < nk; k += 2) {
    stage(std::true_type{}, k, lds_w0, lds_h0, lds_w1, lds_h1);
    stage(std::true_type{}, k + 1, lds_w1, lds_h1, lds_w0, lds_h0);
  }
  // last two stages: nothing left to prefetch (the final fragment reads are unused)
  stage(std::false_type{}, k, lds_w0, lds_h0, lds_w1, lds_h1);
  stage(std::false_type{}, k + 1, lds_w1, lds_h1, lds_w0, lds_h0);
}

template <int NWAVES, int VB16, int NB16, int WI, int HI, bool ATR = false, bool BTR = false>
__device__ __forceinline__ void nt_mainloop(f32x4 (&acc)[VB16][NB16], uint8_t* lds_w0,
                                            uint8_t* lds_w1, uint8_t* lds_h0, uint8_t* lds_h1,
                                            __amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t rh,
                                            const uint32_t (&wgo)[WI], const uint32_t (&hgo)[HI],
                                            int nk, int wave, int lane, int wv, int wt,
                                            uint32_t sa = 0, uint32_t sb = 0) {
  NoHook none;
  nt_mainloop_x<NWAVES, VB16, NB16, WI, HI, ATR, BTR, false>(acc, lds_w0, lds_w1, lds_h0, lds_h1,
                                                             rw, rh, wgo, hgo, nk, wave, lane, wv,
                                                             wt, sa, sb, none);
}

}  // namespace rlk
