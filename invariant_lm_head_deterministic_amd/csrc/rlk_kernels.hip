// HIP kernels of the strict-path selected-token logprob, for gfx950 (MI355X) only.
//
// Numeric contract v3. Every result bit of a row is decided by the rules below and by nothing
// else: not by the row's position in a launch, the launch's row count, the token-tile width,
// the grid, the number of vocab shards, or which CU or XCD ran a block. The pages ask for a
// forward whose inputs, split, merge order, precisions, rounding points and primitives are all
// fixed (RL-Kernel v0.1.0 summary page, "Numeric execution contract"; kongchang.com article,
// "four key links"); these are our choices for each.
//
//  C1 logit. z[t,v] is one fp32 accumulator chain of v_mfma_f32_16x16x32_bf16 steps starting at
//     +0: step i (i = 0 .. H/32-1, ascending) feeds K indices 32i .. 32i+31, lane group g
//     (lanes 16g .. 16g+15) of the instruction carrying 32i+8g .. 32i+8g+7 for both operands.
//     No split-K, no atomics (the ROCm fixes list on the RL-Kernel page: a deterministic
//     MFMA-based GEMM; K-dim reduction and accumulation precision in the boundary table).
//  C2 temperature. z' = z * inv_temperature in fp32 (skipped when it is 1.0f: x * 1.0f == x).
//  C3 vocab split. The vocabulary is S_c contiguous segments of V/S_c; each segment is cut into
//     tiles of 64 columns from its own start, the last one partial (the "actual vocab range"
//     and "local reduction" of the "Linear logprob" boundary row).
//  C4 tile max. m = max of z' over the tile's columns (exact; order-free).
//  C5 tile sum. e(v) = EXP(z'(v) - m). The tile's 64 columns form 4 blocks of 16 (b = 0..3)
//     and 4 lane groups g = 0..3; group g holds the 16 columns 16b + 4g + r, b, r = 0..3 (the
//     MFMA result-register order). Then
//        p[g] = sequential sum of e over (b, r) = (0,0), (0,1), .., (0,3), (1,0), .., (3,3)
//        s    = (p[0] + p[1]) + (p[2] + p[3])
//     Columns past the end of a partial tile contribute exactly +0. (nxbn.cn blog, §3.2 and
//     §4.3: sequential sums inside a thread, then a fixed tree; fp32 intermediates.)
//  C6 entropy term (optional). u uses the same tree with terms e(v) * (z'(v) - m).
//  C7 target ownership. The one tile whose columns contain y_t writes z'[t, y_t] as computed
//     in C1-C2 ("target ownership" in the "Linear logprob" boundary row); nothing is summed.
//  C8 segment fold. M_s = max_j m_j over the segment's tiles. The tiles form groups of 32
//     consecutive tiles from the segment start (the last group partial); inside group q
//        A_q = sequential sum over its tiles j ascending, from +0, of s_j * EXP(m_j - M_s)
//        B_q = sequential sum, from +0, of (u_j + s_j * (m_j - M_s)) * EXP(m_j - M_s)
//     and S_s, U_s are balanced pairwise trees over the groups in index order, padded with +0
//     to a power of two (a pair whose right member is padding passes its left member through).
//  C9 cross-segment merge. M = max_s M_s; S and U are balanced pairwise trees in segment order
//     of S_s * EXP(M_s - M) and (U_s + S_s * (M_s - M)) * EXP(M_s - M) (S_c = 4:
//     (a0 + a1) + (a2 + a3)) — the "cross-rank LSE merge" in a fixed order.
//  C10 outputs. lse = M + LOG(S); logp = z'_y - lse; entropy = LOG(S) - U / S; padded rows
//     (y < 0) write +0; y >= V writes NaN and sets a status bit.
//  C11 primitives (one exp, one log, one rsqrt; the "primitives" item of the contract):
//     EXP(x) = v_exp_f32(x * 0x1.715476p+0f), LOG(x) = v_log_f32(x) * 0x1.62e430p-1f,
//     RSQ(x) = v_rsq_f32(x). Every other operation is one IEEE fp32 operation, rounded to
//     nearest even; the library is built with -ffp-contract=off so nothing is fused (nxbn.cn
//     blog, §3.4 and §4.3).
//  C11p portable primitives (RLK_FLAG_PORTABLE_EXP): EXP, LOG and RSQ are p_exp, p_log and
//     p_rsq below, made of IEEE fp32 operations only, so C1-C12 then fix every output bit as a
//     function of the logits on any IEEE-754 machine, not only on this GPU's transcendental
//     units.
//  C12 RMSNorm (optional). ss = sum of x_k^2 in fp32 — lane l of a 64-wide wave takes the
//     8-element groups l, l+64, l+128, ... in order, sequentially — then a butterfly over lanes
//     with xor distances 32, 16, 8, 4, 2, 1; r = RSQ(ss * fl32(1/H) + eps);
//     y_k = bf16_rne((x_k * r) * gamma_k) (the "RMSNorm" boundary row: reduction domain,
//     epsilon, output boundary; wave64 shuffle steps in a fixed order, nxbn.cn blog §3.2).

#include "rlk_device.h"
#include "rlk_queue.h"

namespace rlk {

// Where a block's work lies: a run of NTPB consecutive vocab tiles of one segment (first global
// column, columns present, global index of the first tile) and a row tile (first row, rows
// present).
struct Tile {
  int64_t start;  // global vocab index of the block's first column
  int len;        // columns present (64 NTPB, or fewer at a segment's end)
  int tile0;      // global tile index of the block's first tile
  int row0;       // first launch row of the row tile
  int rows;       // rows present in the row tile
};

// Row tiles per band: the hidden rows of a band stay under ~64 MB, so they stay in the MALL
// while the band's vocab blocks stream past them.
template <int BT>
__host__ __device__ __forceinline__ int64_t band_row_tiles(int H) {
  const int64_t per = (int64_t)BT * H * 2;
  const int64_t rb = ((int64_t)64 << 20) / per;
  return rb > 0 ? rb : 1;
}

// Blocks of one band of n_tt_band row tiles, rounded up to a multiple of the 8 XCDs.
__host__ __device__ __forceinline__ int64_t band_blocks(int64_t n_vb, int64_t n_tt_band) {
  return (n_vb * n_tt_band + 7) / 8 * 8;
}

// The columns and rows of vocab block vb (NTPB tiles of one segment) and row tile tt.
template <int BT, int NTPB>
__device__ __forceinline__ void set_tile(const LmheadArgs& a, int vb, int tt, Tile& t) {
  const int bps = (a.tiles_per_seg + NTPB - 1) / NTPB;
  const int seg = a.seg_begin + vb / bps;
  const int jb = vb % bps;
  const int64_t col0 = (int64_t)jb * NTPB * kVocabTile;
  // uniform by construction; readfirstlane states that to the compiler
  t.start = uni64((int64_t)seg * a.seg_len + col0);
  t.len = uni((int)min((int64_t)NTPB * kVocabTile, a.seg_len - col0));
  t.tile0 = uni(seg * a.tiles_per_seg + jb * NTPB);
  t.row0 = uni(tt * BT);
  t.rows = uni(min(BT, a.rows - tt * BT));
}

// Block -> (vocab block, row tile), XCD-aware. Row tiles go in bands (band_row_tiles), one band
// after the other in block order; inside a band, consecutive block ids go round-robin to the 8
// XCDs, so they are remapped so that each XCD walks a contiguous range of the band's items, a
// group of 8 vocab blocks at a time across the band's row tiles (W and hidden tiles shared in L2;
// 8 was the best of 2, 4, 8, 16 measured on the Qwen3-8B head). Returns false for the few
// padding blocks.
template <int BT, int NTPB>
__device__ __forceinline__ bool map_tile(const LmheadArgs& a, Tile& t) {
  const int bps = (a.tiles_per_seg + NTPB - 1) / NTPB;  // vocab blocks per segment
  const int n_vb = a.n_seg * bps;
  const int n_tt = (a.rows + BT - 1) / BT;
  const int64_t rb = band_row_tiles<BT>(a.H);
  const int64_t full = band_blocks(n_vb, rb);  // blocks of a full band
  const int64_t band = (int64_t)blockIdx.x / full;
  const int64_t bid = (int64_t)blockIdx.x - band * full;
  const int tt0 = (int)(band * rb);
  if (tt0 >= n_tt) return false;
  const int nb_tt = (int)min((int64_t)n_tt - tt0, rb);  // row tiles of this band
  const int64_t nblk = band_blocks(n_vb, nb_tt);
  if (bid >= nblk) return false;
  const int64_t n_items = (int64_t)n_vb * nb_tt;
  const int64_t per_xcd = nblk / 8;
  const int64_t L = (bid % 8) * per_xcd + bid / 8;
  if (L >= n_items) return false;
  constexpr int GV = 8;
  const int64_t grp = L / ((int64_t)GV * nb_tt);
  const int first_v = (int)(grp * GV);
  const int gsz = min(GV, n_vb - first_v);
  const int64_t within = L - grp * GV * nb_tt;
  const int vb = first_v + (int)(within % gsz);
  const int tt = tt0 + (int)(within / gsz);
  set_tile<BT, NTPB>(a, vb, tt, t);
  return true;
}

// Hands out one item of queue x (the count of items handed out from it before).
__device__ __forceinline__ uint32_t claim(uint32_t* q, int x) {
  return __hip_atomic_fetch_add(q + x, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The item behind claim count c of queue (xq + qi) mod 8; a drained queue moves the block on to
// the next queue (qi + 1), and false means that all eight are drained. Ends after at most eight
// claims.
__device__ __forceinline__ bool next_item(const LmheadArgs& a, int xq, int& qi, uint32_t c,
                                          int& vb, int& tt) {
  while (true) {
    if (queue_item(a, (xq + qi) & (kQueues - 1), c, vb, tt)) return true;
    if (++qi == kQueues) return false;
    c = claim(a.queue, (xq + qi) & (kQueues - 1));
  }
}

// MFMA layout (v_mfma_f32_16x16x32_bf16, vocab = MFMA rows from W, tokens = MFMA columns from
// the hidden states): an operand fragment is 16 rows x 32 K, lane l holding row l & 15 and the
// 8 K elements 8 (l >> 4) .. +7; the result block gives lane l the token l & 15 and the 4 vocab
// rows 4 (l >> 4) + r. A wave owns VB16 vocab blocks and NB16 token blocks of 16.

// Target of this lane's token in token block j (-1 past the row tile), read before the K loop so
// that its latency hides behind the MFMAs.
template <int NB16>
__device__ __forceinline__ void load_targets(int (&y)[NB16], const LmheadArgs& a, const Tile& t,
                                             int wt, int lane) {
#pragma unroll
  for (int j = 0; j < NB16; ++j) {
    const int rr = 16 * (wt * NB16 + j) + (lane & 15);
    y[j] = rr < t.rows ? a.targets[t.row0 + rr] : -1;
  }
}

// Reductions across the lane groups of C5 with gfx950's lane-swap instructions (VALU, no LDS):
// v_permlane16_swap exchanges rows 1 <-> 0 and 3 <-> 2 of 16 lanes between its two operands,
// v_permlane32_swap the two halves, so with x in both operands every lane gets its own value
// and its partner's (lane ^ 16, lane ^ 32), always as (even row, odd row) / (low, high): the
// sum and the max below are the C5 tree ((p0 + p1) + (p2 + p3)) on every lane.
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// One tile (C4-C7) for one token block: z holds this lane's 16 values of the tile (block b,
// register r at 4 b + r; column 16 b + 4 g + r). MASK: the tile is a segment's partial last
// tile of tlen columns.
template <bool MASK, bool ENT, bool PORT>
__device__ __forceinline__ void tile_one(const float (&z)[16], int g, int tlen, float& m_out,
                                         float& s_out, float& u_out) {
  float mm = -INFINITY;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int col = 16 * (q >> 2) + 4 * g + (q & 3);
    if (!MASK || col < tlen) mm = fmaxf(mm, z[q]);
  }
  const float m = max_xor32(max_xor16(mm));
  float ps = 0.0f, pq = 0.0f;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int col = 16 * (q >> 2) + 4 * g + (q & 3);
    const float d = z[q] - m;
    float e = EXP<PORT>(d);
    if (MASK && col >= tlen) e = 0.0f;
    ps = ps + e;
    if constexpr (ENT) {
      float qq = e * d;
      if (MASK && col >= tlen) qq = 0.0f;
      pq = pq + qq;
    }
  }
  m_out = m;
  s_out = sum_xor32(sum_xor16(ps));
  u_out = ENT ? sum_xor32(sum_xor16(pq)) : 0.0f;
}

// Fused tile epilogue (C2, C4-C7) on the MFMA result registers of one wave. The wave owns vocab
// blocks 16 (VB16 wv + i) .. of the block, i.e. VB16/4 whole tiles, and token blocks
// 16 (NB16 wt + j) .., so every reduction of a tile stays inside the wave: a lane-local
// sequential sum plus two exchanges between lane groups.
template <int VB16, int NB16, bool ENT, bool TEMP, bool PORT>
__device__ __forceinline__ void tile_epilogue(f32x4 (&acc)[VB16][NB16], const int (&ytgt)[NB16],
                                              const LmheadArgs& a, const Tile& t, int wv, int wt,
                                              int lane) {
  static_assert(VB16 % 4 == 0, "a wave owns whole tiles");
  const int g = lane >> 4;
  if constexpr (TEMP) {
#pragma unroll
    for (int i = 0; i < VB16; ++i)
#pragma unroll
      for (int j = 0; j < NB16; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = acc[i][j][r] * a.inv_tau;
  }
#pragma unroll
  for (int c = 0; c < VB16 / 4; ++c) {
    const int tc = wv * (VB16 / 4) + c;  // tile index inside the block
    const int tlen = min(kVocabTile, t.len - tc * kVocabTile);
    if (tlen <= 0) continue;  // past the segment's end (uniform across the wave)
    const int64_t go = (int64_t)(t.tile0 + tc - a.g_base) * a.ld;
    const int64_t tstart = t.start + (int64_t)tc * kVocabTile;
#pragma unroll
    for (int j = 0; j < NB16; ++j) {
      float z[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) z[q] = acc[4 * c + (q >> 2)][j][q & 3];
      float m, sum, u;
      if (tlen == kVocabTile) tile_one<false, ENT, PORT>(z, g, tlen, m, sum, u);
      else tile_one<true, ENT, PORT>(z, g, tlen, m, sum, u);
      const int rr = 16 * (wt * NB16 + j) + (lane & 15);  // row inside the row tile
      if (g == 0 && rr < t.rows) {
        const int64_t row = (int64_t)t.row0 + rr;
        a.part_m[go + row] = m;
        a.part_s[go + row] = sum;
        if constexpr (ENT) a.part_u[go + row] = u;
      }
      // target ownership: the lane whose registers hold column y_t of this tile writes z'[t, y_t]
      const int y = ytgt[j];
      const int64_t d = (int64_t)y - tstart;
      const bool in_tile = y >= 0 && d >= 0 && d < tlen;
      const int dd = (int)d;
      const bool mine = in_tile && (((dd >> 2) & 3) == g);
      if (__any(mine)) {
        const int ridx = (dd >> 4) * 4 + (dd & 3);
        float v = 0.0f;
#pragma unroll
        for (int q = 0; q < 16; ++q) v = (q == ridx) ? z[q] : v;
        if (mine) a.tgt[t.row0 + rr] = v;
      }
    }
  }
}

// Direct-to-LDS staging of tile t: DMA instruction q of a wave fills the 8 staged rows from
// 8 (q NWAVES + wave); lane l writes position l & 7 of row (l >> 3) of that group, so it loads
// the logical piece that the swizzle puts there. Rows past the tile or the launch are clamped to
// the last valid row (their results are never used), so every address lies inside the tile's
// descriptor. The per-lane byte offsets are fixed; the K stage is the scalar offset.
template <int NWAVES, int WI, int HI>
__device__ __forceinline__ void stage_operands(const LmheadArgs& a, const Tile& t, int wave,
                                               int lane, uint32_t (&wgo)[WI], uint32_t (&hgo)[HI],
                                               __amdgpu_buffer_rsrc_t& rw,
                                               __amdgpu_buffer_rsrc_t& rh) {
  const int H = a.H;
#pragma unroll
  for (int q = 0; q < WI; ++q) {
    const int r = 8 * (q * NWAVES + wave) + (lane >> 3);
    const int c = (lane & 7) ^ swz(r);
    wgo[q] = (uint32_t)(min(r, t.len - 1) * H + c * 8) * 2u;
  }
#pragma unroll
  for (int q = 0; q < HI; ++q) {
    const int r = 8 * (q * NWAVES + wave) + (lane >> 3);
    const int c = (lane & 7) ^ swz(r);
    hgo[q] = (uint32_t)(min(r, t.rows - 1) * H + c * 8) * 2u;
  }
  rw = make_rsrc(a.W + (t.start - a.w_row0) * (int64_t)H, t.len * H * 2);
  rh = make_rsrc(a.hidden + (int64_t)t.row0 * H, t.rows * H * 2);
}

// --------------------------------------------------------------------------------------------
// K1: LM-head tile kernel. One item = 4 vocab tiles (256 columns of one segment) x BT rows.
// Waves: VW split the item's columns, TW split the rows; each wave owns VB16 = 16 / VW vocab
// blocks x NB16 = 2 NTB token blocks of 16 as 16x16 MFMA result tiles (vocab = MFMA rows, tokens
// = MFMA columns), i.e. whole tiles for its rows, so the epilogue needs no LDS.
// Persistent: one block per CU takes items from its XCD's queue (queue_item), then from the
// other XCDs' queues, so a CU that the power limit clocks lower simply takes fewer items, and
// the first K stages of the next item load while the current one runs its epilogue. Which block
// computes an item never changes its arithmetic, so the bits do not depend on the schedule.
// --------------------------------------------------------------------------------------------
template <int VW, int TW, int NTB, bool ENT, bool TEMP, bool PORT>
__global__ void __launch_bounds__(64 * VW * TW)
k_lmhead(const LmheadArgs a) {
  constexpr int NWAVES = VW * TW;
  constexpr int BT = 32 * NTB * TW;
  constexpr int BW = 4 * kVocabTile;          // block columns: 4 tiles
  constexpr int VB16 = BW / 16 / VW;          // vocab blocks of 16 per wave
  constexpr int NB16 = 2 * NTB;               // token blocks of 16 per wave
  constexpr int WI = BW / 8 / NWAVES;          // DMA instructions per wave per W stage
  constexpr int HI = BT / 8 / NWAVES;          // DMA instructions per wave per hidden stage
  static_assert(VB16 * VW * 16 == BW && WI * 8 * NWAVES == BW && HI * 8 * NWAVES == BT, "tiling");

  // two stages as distinct objects, so the compiler can tell a DMA into one stage from reads
  // of the other and does not wait for the DMA before those reads
  __shared__ __attribute__((aligned(1024))) uint8_t lds_w0[BW * kRowBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_w1[BW * kRowBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_h0[BT * kRowBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_h1[BT * kRowBytes];

  // the block's next item (vocab block, row tile), -1 when every queue is drained, and the
  // queue offset of its claims (from this XCD's queue); written by thread 0, read after barriers
  __shared__ int s_next[2];
  __shared__ int s_qi;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wv = wave % VW;
  const int wt = wave / VW;
  const int nk = a.H / kKStage;  // even: H is a multiple of 128
  const bool leader = tid == 0;
  // this XCD's queue: the XCC_ID hardware register (all 32 bits; the id is bits 3:0)
  auto xcc_queue = []() { return (int)(__builtin_amdgcn_s_getreg((31 << 11) | 20) & (kQueues - 1)); };
  // The arguments again from the kernel-argument segment (a is the kernel's only argument, at
  // offset 0), by scalar loads through a pointer the compiler cannot see through: what the tile
  // boundary needs is then loaded there instead of held in scalar registers across the K loop,
  // which has none to spare. (Taking a's address instead would copy it to private memory.)
  typedef const __attribute__((address_space(4))) LmheadArgs* kargs_t;
  auto args = []() -> const LmheadArgs& {
    uint64_t p = (uint64_t)__builtin_amdgcn_kernarg_segment_ptr();
    __asm__ volatile("" : "+s"(p));
    return *(const LmheadArgs*)(kargs_t)p;
  };
  uint32_t pend = 0;  // thread 0: claim count in flight for the next item

  if (leader) {
    const int xq = xcc_queue();
    int qi = 0, vb = -1, tt = 0;
    if (!next_item(a, xq, qi, claim(a.queue, xq), vb, tt)) vb = -1;
    s_next[0] = vb;
    s_next[1] = tt;
    s_qi = qi;
  }
  __syncthreads();
  if (uni(s_next[0]) >= 0) {
    Tile t;
    set_tile<BT, 4>(a, uni(s_next[0]), uni(s_next[1]), t);
    uint32_t wgo[WI], hgo[HI];
    __amdgpu_buffer_rsrc_t rw, rh;
    stage_operands<NWAVES, WI, HI>(a, t, wave, lane, wgo, hgo, rw, rh);
    issue_stage<NWAVES, WI, HI>(rw, rh, wgo, hgo, 0, lds_w0, lds_h0, wave);
    issue_stage<NWAVES, WI, HI>(rw, rh, wgo, hgo, 1, lds_w1, lds_h1, wave);
    if (leader) pend = claim(a.queue, (xcc_queue() + s_qi) & (kQueues - 1));
    // Tile loop. The next item is resolved at the start of this tile's K loop (its claim went
    // out one tile earlier); once every wave is past this tile's last fragment read, the first
    // two K stages of the next tile are issued, and only then does this tile's epilogue run.
    while (true) {
      f32x4 acc[VB16][NB16];
#pragma unroll
      for (int i = 0; i < VB16; ++i)
#pragma unroll
        for (int j = 0; j < NB16; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.0f;
      auto resolve = [&]() {
        if (leader) {
          int qi = s_qi, nv = -1, nt = 0;
          if (!next_item(args(), xcc_queue(), qi, pend, nv, nt)) nv = -1;
          s_next[0] = nv;
          s_next[1] = nt;
          s_qi = qi;
        }
      };
      nt_mainloop_x<NWAVES, VB16, NB16, WI, HI, false, false, true>(
          acc, lds_w0, lds_w1, lds_h0, lds_h1, rw, rh, wgo, hgo, nk, wave, lane, wv, wt, 0u, 0u,
          resolve);
      __syncthreads();
      const LmheadArgs& b = args();
      // an opaque copy of the lane id: what the boundary and the epilogue derive from it is
      // computed here, not hoisted out of the tile loop and held across the K loop
      int ln = lane;
      __asm__ volatile("" : "+v"(ln));
      // the targets of the wave's rows are read only now: held across the K loop they cost
      // the registers that the loop needs for two waves per SIMD (measured: 4% slower)
      int ytgt[NB16];
      load_targets<NB16>(ytgt, b, t, wt, ln);
      const int nv = uni(s_next[0]);
      if (nv >= 0) {
        Tile tn;
        set_tile<BT, 4>(b, nv, uni(s_next[1]), tn);
        stage_operands<NWAVES, WI, HI>(b, tn, wave, ln, wgo, hgo, rw, rh);
        issue_stage<NWAVES, WI, HI>(rw, rh, wgo, hgo, 0, lds_w0, lds_h0, wave);
        issue_stage<NWAVES, WI, HI>(rw, rh, wgo, hgo, 1, lds_w1, lds_h1, wave);
        if (leader) pend = claim(b.queue, (xcc_queue() + s_qi) & (kQueues - 1));
      }
      tile_epilogue<VB16, NB16, ENT, TEMP, PORT>(acc, ytgt, b, t, wv, wt, ln);
      if (nv < 0) break;
      // the next tile again from its item, rather than held across the epilogue
      __asm__ volatile("" ::: "memory");
      set_tile<BT, 4>(args(), uni(s_next[0]), uni(s_next[1]), t);
    }
  }
  // the last block of the launch to get here resets the queues for the next launch
  if (leader && claim(a.queue, kQueues) == gridDim.x - 1) {
    for (int x = 0; x <= kQueues; ++x)
      __hip_atomic_exchange(a.queue + x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// --------------------------------------------------------------------------------------------
// K1d: deep-pipeline LM-head tile kernel for launches of few rows (decode batches). Same MFMA
// chain (C1), same fragment order and the same per-tile epilogue as k_lmhead, hence the same
// bits; only the staging depth and the block shape (NTPB = 3 or 4 tiles) differ. A decode
// batch has one row tile, so a launch has few blocks and the W stream is bound by the bytes
// each block keeps in flight: these variants cycle NS (2-4) LDS stages, so NS-1 stages of DMA
// are outstanding while one is read.
// HS > 0: W streams through its own ring of NS stages and the hidden rows through a ring of HS
// (they are L2-resident and arrive quickly), so the same LDS holds more W in flight. Measured
// per vocab segment: 193-256 rows 106 -> 92 us (3 + 2 stages), 65-128 rows with 6 waves
// 74 -> 73 us (4 + 3); slower at <= 64 rows with a ring of 2 for the hidden rows, whose short
// stages leave those too little time, and for 65-192 rows with 12 waves (one ring of 3 stages:
// 70-80 us; 4 + 2 stages: 77-84 us).
// NB16 (token blocks of 16 per wave) may be odd: 12 waves of 48 rows cover 192.
// The stage buffer is picked at run time; the DMA is issued from inline assembly so that the
// compiler, which cannot tell the stage buffers apart at run time, does not wait for every
// outstanding DMA before each LDS read. Its completion is awaited explicitly (vmcnt) before the
// barrier that publishes a stage, exactly as in k_lmhead.
// --------------------------------------------------------------------------------------------
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor (base, unstrided, `bytes` long, 32-bit data format) in 4 SGPRs.
__device__ __forceinline__ i32x4 buffer_desc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  // the descriptor is uniform by construction; readfirstlane keeps it in SGPRs, which the
  // inline assembly below requires
  i32x4 d;
  d[0] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)b);
  d[1] = __builtin_amdgcn_readfirstlane((int32_t)((uint32_t)(b >> 32) & 0xffffu));
  d[2] = __builtin_amdgcn_readfirstlane((int32_t)bytes);
  d[3] = 0x00020000;
  return d;
}

// buffer_load_dwordx4 ... lds: lane l's 16 bytes at voff + soff land at LDS byte lds_addr + 16 l.
__device__ __forceinline__ void dma16_asm(i32x4 desc, uint32_t lds_addr, uint32_t voff,
                                          uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(desc), "s"(soff)
               : "memory");
}

template <int D>
__device__ __forceinline__ void wait_vm() {
  __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(D) : "memory");
}

template <int VW, int TW, int NB16, int NS, int NTPB, int HS, bool ENT, bool TEMP, bool PORT>
__global__ void __launch_bounds__(64 * VW * TW) k_lmhead_deep(const LmheadArgs a) {
  // NB16: token blocks of 16 per wave
  constexpr int NWAVES = VW * TW;
  constexpr int BT = 16 * NB16 * TW;
  constexpr int BW = NTPB * kVocabTile;  // block columns
  constexpr int VB16 = BW / 16 / VW;     // vocab blocks of 16 per wave
  constexpr int WI = BW / 8 / NWAVES;
  // hidden rows are staged in whole DMA rounds of 8 NWAVES rows; rows past BT repeat the last
  // row and are never read
  constexpr int HI = (BT / 8 + NWAVES - 1) / NWAVES;
  constexpr int DPS = WI + HI;  // DMA instructions per wave per stage
  constexpr int SW = BW * kRowBytes;
  constexpr int SH = 8 * HI * NWAVES * kRowBytes;
  static_assert(VB16 * VW * 16 == BW && VB16 % 4 == 0 && WI * 8 * NWAVES == BW && BT % 32 == 0,
                "tiling");
  static_assert(NS >= 2 && NS <= 6 && (NS - 2) * DPS <= 63 && (NS - 1) * (HI + WI) <= 63,
                "stages");
  constexpr bool SPLIT = HS > 0;      // separate rings for W and the hidden rows
  constexpr int NSH = SPLIT ? HS : NS;  // stages of the hidden rows' ring
  static_assert(!SPLIT || (HS >= 2 && HS < NS), "rings");

  __shared__ __attribute__((aligned(1024))) uint8_t lds_w[NS * SW];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_h[NSH * SH];

  Tile t;
  if (!map_tile<BT, NTPB>(a, t)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wv = wave % VW;
  const int wt = wave / VW;
  int ytgt[NB16];
  load_targets<NB16>(ytgt, a, t, wt, lane);
  const int H = a.H;
  const uint16_t* __restrict__ Wt = a.W + (t.start - a.w_row0) * (int64_t)H;
  const uint16_t* __restrict__ Ht = a.hidden + (int64_t)t.row0 * H;

  uint32_t wgo[WI], hgo[HI];
#pragma unroll
  for (int q = 0; q < WI; ++q) {
    const int r = 8 * (q * NWAVES + wave) + (lane >> 3);
    const int c = (lane & 7) ^ swz(r);
    wgo[q] = (uint32_t)(min(r, t.len - 1) * H + c * 8) * 2u;
  }
#pragma unroll
  for (int q = 0; q < HI; ++q) {
    const int r = 8 * (q * NWAVES + wave) + (lane >> 3);
    const int c = (lane & 7) ^ swz(r);
    hgo[q] = (uint32_t)(min(r, t.rows - 1) * H + c * 8) * 2u;
  }
  const i32x4 dw = buffer_desc(Wt, (uint32_t)(t.len * H * 2));
  const i32x4 dh = buffer_desc(Ht, (uint32_t)(t.rows * H * 2));
  const uint32_t lw0 = (uint32_t)(uintptr_t)lds_w + 8 * wave * kRowBytes;
  const uint32_t lh0 = (uint32_t)(uintptr_t)lds_h + 8 * wave * kRowBytes;
  const int nk = H / kKStage;
  auto issue_w = [&](int kc) {
    const int b = kc % NS;
    const uint32_t so = (uint32_t)kc * kRowBytes;
#pragma unroll
    for (int q = 0; q < WI; ++q)
      dma16_asm(dw, lw0 + b * SW + 8 * q * NWAVES * kRowBytes, wgo[q], so);
  };
  auto issue_h = [&](int kc) {
    const int b = kc % NSH;
    const uint32_t so = (uint32_t)kc * kRowBytes;
#pragma unroll
    for (int q = 0; q < HI; ++q)
      dma16_asm(dh, lh0 + b * SH + 8 * q * NWAVES * kRowBytes, hgo[q], so);
  };
  auto issue = [&](int kc) {
    issue_w(kc);
    issue_h(kc);
  };

  f32x4 acc[VB16][NB16];
#pragma unroll
  for (int i = 0; i < VB16; ++i)
#pragma unroll
    for (int j = 0; j < NB16; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.0f;

  // sub-step s (K 32s .. 32s+31 of a stage): piece 4s + (lane >> 4) of row lane & 15 of each
  // 16-row block (one lane offset per sub-step serves every block, see k_lmhead)
  const int r16 = lane & 15;
  int loff[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) loff[s] = r16 * kRowBytes + (((4 * s + (lane >> 4)) ^ swz(r16)) << 4);
  const int a0 = 16 * wv * VB16 * kRowBytes, b0 = 16 * wt * NB16 * kRowBytes;
  bf16x8 fa[2][VB16], fb[2][NB16];
  auto load_frags = [&](int kst, int s, int slot) {  // sub-step s of K stage kst
    const uint8_t* pa = lds_w + (kst % NS) * SW + a0 + loff[s];
    const uint8_t* pb = lds_h + (kst % NSH) * SH + b0 + loff[s];
#pragma unroll
    for (int j = 0; j < NB16; ++j) fb[slot][j] = *(const bf16x8*)(pb + j * 16 * kRowBytes);
#pragma unroll
    for (int i = 0; i < VB16; ++i) fa[slot][i] = *(const bf16x8*)(pa + i * 16 * kRowBytes);
  };
  auto mfmas = [&](int slot) {
#pragma unroll
    for (int i = 0; i < VB16; ++i)
#pragma unroll
      for (int j = 0; j < NB16; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[slot][i], fb[slot][j], acc[i][j],
                                                            0, 0, 0);
  };
  // wait until the DMA of stage k+1 is done while up to `later` younger stages stay in flight
  auto wait_stage = [&](int later) {
    if constexpr (NS >= 4) {
      if (later >= 2) { wait_vm<2 * DPS>(); return; }
    }
    if constexpr (NS >= 3) {
      if (later >= 1) { wait_vm<DPS>(); return; }
    }
    wait_vm<0>();
  };

  if constexpr (SPLIT) {
    // Issue order: stage by stage, H(j) (j < HS) then W(j) (j < NS); after the barrier of stage
    // k, H(k+HS) and W(k+NS). Loads complete in issue order, so waiting for H(k+1) leaves in
    // flight only what was issued after it: W(k+1-HS+NS) and the HS-2 later stages' pairs.
    // W stage k+NS then has NS-1 stages of time to land, the hidden rows' stage k+HS HS-1.
    for (int j = 0; j < NS && j < nk; ++j) {
      if (j < HS) issue_h(j);
      issue_w(j);
    }
    if (nk >= NS) wait_vm<(HS - 1) * HI + (NS - 1) * WI>();  // H0 and W0 have landed
    else wait_vm<0>();
    __syncthreads();
    load_frags(0, 0, 0);
    for (int k = 0; k < nk; ++k) {
      mfmas(0);
      load_frags(k, 1, 1);
      if (k - 1 + NS < nk) wait_vm<WI + (HS - 2) * (HI + WI)>();
      else wait_vm<0>();
      __syncthreads();
      if (k + HS < nk) issue_h(k + HS);  // into stage k's buffers, free after the barrier
      if (k + NS < nk) issue_w(k + NS);
      mfmas(1);
      load_frags(k + 1, 0, 0);
    }
  } else {
    // prologue: stages 0 .. NS-1 in flight, wait for stage 0
    const int pro = nk < NS ? nk : NS;
    for (int j = 0; j < pro; ++j) issue(j);
    wait_stage(pro - 1 > NS - 2 ? NS - 2 : pro - 1);
    // (the youngest pro-1 stages may still be in flight; stage 0 has landed for this wave)
    __syncthreads();
    load_frags(0, 0, 0);
    for (int k = 0; k < nk; ++k) {
      mfmas(0);
      load_frags(k, 1, 1);
      // stage k+1 must have landed for every wave; stages k+2 .. k+NS-1 may stay in flight
      const int issued_last = (k - 1 + NS < nk - 1 ? k - 1 + NS : nk - 1);  // newest issued
      wait_stage(issued_last - (k + 1));
      __syncthreads();
      if (k + NS < nk) issue(k + NS);  // into stage k's buffer, free after the barrier
      mfmas(1);
      load_frags(k + 1, 0, 0);
    }
  }
  wait_vm<0>();

  tile_epilogue<VB16, NB16, ENT, TEMP, PORT>(acc, ytgt, a, t, wv, wt, lane);
}

// --------------------------------------------------------------------------------------------
// K1s: streaming LM-head kernel for decode launches of at most 16 rows (32 when H is not a
// multiple of 256). Same MFMA chain (C1), fragment order and per-tile epilogue as k_lmhead, hence
// the same bits.
//
// A decode launch is bound by the W stream: every W row is used by at most 256 rows. Loads
// complete in issue order per wave, so a wave that waits for a recent load also waits for every
// older one; kernels whose waves both stream W and read the hidden rows keep W only as deep in
// flight as the hidden rows. Here the two streams come from different waves:
//  - NPW producer waves only copy W into a ring of NS LDS stages (64 W rows x 64 K each), keeping
//    NS-1 stages in flight and waiting, before each stage's barrier, only for their own copy of
//    that stage;
//  - 4 compute waves read the stage's W fragments from LDS and their own hidden rows straight
//    from memory into registers (the rows of a decode batch stay in L2), HD stages ahead.
// One block per CU; an item is one 64-column tile with all the launch's rows (wave w owns token
// blocks NBW w .. NBW w + NBW - 1), so a CU streams whole tiles one after the other without
// draining its ring between them, and every CU of the device takes part. Block b takes the
// items b, b + G, b + 2G, ... of the launch (G blocks).
// --------------------------------------------------------------------------------------------

// f(integral_constant<int, S>) for each S of the sequence, in order.
template <class F, int... S>
__device__ __forceinline__ void unroll_seq(std::integer_sequence<int, S...>, F&& f) {
  (f(std::integral_constant<int, S>{}), ...);
}

// s_waitcnt vmcnt(n * D) for a run-time n in [0, N] (one branch per value).
template <int D, int N>
__device__ __forceinline__ void wait_vm_n(int n) {
  if constexpr (N == 0) {
    wait_vm<0>();
  } else {
    if (n >= N) wait_vm<N * D>();
    else wait_vm_n<D, N - 1>(n);
  }
}

template <int CW, int NBW, int SK, int NS, int NPW, int HD, bool ENT, bool TEMP, bool PORT>
__global__ void __launch_bounds__(64 * (CW + NPW)) k_lmhead_stream(const LmheadArgs a) {
  constexpr int RB = 2 * SK;                // bytes of one staged W row
  constexpr int SW = kVocabTile * RB;       // bytes of one W stage (64 rows x SK of K)
  constexpr int DPS = SW / 1024;            // DMA instructions per stage (1 KB each)
  constexpr int DPW = DPS / NPW;            // ... per producer wave
  constexpr int KS = SK / 32;               // MFMA K-steps per stage
  constexpr int RPI = 1024 / RB;            // staged rows per DMA instruction
  static_assert((SK == 128 || SK == 256) && NPW * DPW == DPS && NS >= 3 && (NS - 2) * DPW <= 63,
                "stages");
  static_assert(HD >= 1, "hidden prefetch");
  __shared__ __attribute__((aligned(1024))) uint8_t lds_w[NS * SW];
  // Staged rows of RB = 256 or 512 bytes: piece c (16 bytes) of row r sits at position
  // c ^ (r & 15), so a fragment read (16 consecutive rows, one piece each) covers the 64 banks
  // once.

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int H = a.H;
  const int nk = H / SK;  // the launcher picks SK dividing H
  const int n_items = a.n_seg * a.tiles_per_seg;
  const int G = (int)gridDim.x;
  const int my_items = (n_items - (int)blockIdx.x + G - 1) / G;
  const int total = my_items * nk;  // stages this block streams
  // the columns of the block's i-th item
  auto item_tile = [&](int i, Tile& t) {
    const int it = (int)blockIdx.x + i * G;
    const int seg = a.seg_begin + it / a.tiles_per_seg;
    const int jt = it % a.tiles_per_seg;
    const int64_t col0 = (int64_t)jt * kVocabTile;
    t.start = uni64((int64_t)seg * a.seg_len + col0);
    t.len = uni((int)min((int64_t)kVocabTile, a.seg_len - col0));
    t.tile0 = uni(seg * a.tiles_per_seg + jt);
    t.row0 = 0;
    t.rows = a.rows;
  };

  if (wave >= CW) {
    // ---- producer: W stages into the ring ----
    const int p = wave - CW;
    const uint32_t lbase = (uint32_t)(uintptr_t)lds_w;
    int i_item = 0, k_in = 0;  // next stage to issue: item, K stage
    i32x4 desc;
    uint32_t voff[DPW];
    auto set_item = [&](int i) {
      Tile t;
      item_tile(i, t);
      desc = buffer_desc(a.W + (t.start - a.w_row0) * (int64_t)H, (uint32_t)(t.len * H * 2));
#pragma unroll
      for (int d = 0; d < DPW; ++d) {
        const int q = d * NPW + p;  // instruction q fills staged rows RPI q .. RPI q + RPI - 1
        const int r = RPI * q + lane / (RB / 16);
        const int c = (lane % (RB / 16)) ^ (r & 15);
        voff[d] = (uint32_t)(min(r, t.len - 1) * H + c * 8) * 2u;
      }
    };
    auto issue = [&](int g) {  // global stage g = (i_item, k_in)
      if (k_in == 0) set_item(i_item);
      // uniform by construction; readfirstlane keeps the asm's scalar operands in SGPRs
      const uint32_t dst = (uint32_t)uni((int)(lbase + (uint32_t)(g % NS) * SW));
      const uint32_t so = (uint32_t)uni(k_in * RB);
      i32x4 du;
#pragma unroll
      for (int w = 0; w < 4; ++w) du[w] = uni(desc[w]);
#pragma unroll
      for (int d = 0; d < DPW; ++d)
        dma16_asm(du, dst + (uint32_t)(d * NPW + p) * 1024u, voff[d], so);
      if (++k_in == nk) {
        k_in = 0;
        ++i_item;
      }
    };
    const int pro = min(NS - 1, total);
    for (int g = 0; g < pro; ++g) issue(g);
    for (int g = 0; g < total; ++g) {
      // stage g has landed (for this wave) once at most the younger stages are in flight
      wait_vm_n<DPW, NS - 2>(min(NS - 2, total - 1 - g));
      __asm__ volatile("s_barrier" ::: "memory");
      // the slot of stage g - 1 is free: every compute wave finished it before this barrier
      if (g + NS - 1 < total) issue(g + NS - 1);
    }
    return;
  }

  // ---- compute waves ----
  const int rows = a.rows;
  const bool has_rows = 16 * NBW * wave < rows;  // uniform: this wave owns a row of the launch
  // hidden fragment of token block j (row 16 (NBW wave + j) + lane & 15, clamped into the launch)
  // at K-step s of stage k: lane group lane >> 4 carries K SK k + 32 s + 8 (lane >> 4) .. +7
  uint32_t hoff[NBW];
#pragma unroll
  for (int j = 0; j < NBW; ++j) {
    const int r = min(16 * (NBW * wave + j) + (lane & 15), rows - 1);
    hoff[j] = (uint32_t)(r * H + 8 * (lane >> 4)) * 2u;
  }
  const uint8_t* hbase = (const uint8_t*)a.hidden;
  bf16x8 hb[HD + 1][KS][NBW];
  // always issued (rows are clamped into the launch), so that the compiler's count of
  // outstanding loads stays exact and each wait covers only the stage it needs
  auto load_h = [&](auto slot_c, int k) __attribute__((always_inline)) {  // slot: compile-time
    constexpr int slot = decltype(slot_c)::value;
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int j = 0; j < NBW; ++j)
        hb[slot][s][j] = *(const bf16x8*)(hbase + hoff[j] + (uint32_t)(SK * k + 32 * s) * 2u);
  };
  // fragment read of K-step s: row lane & 15 of a 16-row block, logical piece 4 s + (lane >> 4)
  const int r16 = lane & 15;
  int loff[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) loff[s] = r16 * RB + (((4 * s + (lane >> 4)) ^ r16) << 4);

  f32x4 acc[4][NBW];
  int ytgt[NBW];
  int kp = 0;  // K stage of the next hidden prefetch
  unroll_seq(std::make_integer_sequence<int, HD>{}, [&](auto hc) __attribute__((always_inline)) {
    load_h(hc, kp);
    if (++kp == nk) kp = 0;
  });
  int item = 0, k = 0;
  Tile t;
  item_tile(0, t);
  // The stage loop, unrolled HD + 1 times so that the hidden ring's slots are compile-time.
  auto step = [&](auto slot_c, int g) __attribute__((always_inline)) {
    constexpr int slot = decltype(slot_c)::value;
    if (k == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.0f;
      // the item's targets, read now so that they have long landed at its epilogue
      load_targets<NBW>(ytgt, a, t, wave, lane);
    }
    // every LDS read of the previous stage is done before its slot is handed back
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // hidden rows HD stages ahead (the same rows for every item: K wraps at the item's end;
    // past the block's last stage the loads are harmless repeats)
    load_h(std::integral_constant<int, (slot + HD) % (HD + 1)>{}, kp);
    if (++kp == nk) kp = 0;
    if (has_rows) {
      const uint8_t* sp = lds_w + (g % NS) * SW;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        bf16x8 fa[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[i] = *(const bf16x8*)(sp + i * 16 * RB + loff[s]);
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], hb[slot][s][j], acc[i][j],
                                                                0, 0, 0);
      }
    }
    if (++k == nk) {
      if (has_rows) tile_epilogue<4, NBW, ENT, TEMP, PORT>(acc, ytgt, a, t, 0, wave, lane);
      k = 0;
      if (++item < my_items) item_tile(item, t);
    }
  };
  constexpr auto seq = std::make_integer_sequence<int, HD + 1>{};
  int g = 0;
  for (; g + HD < total; g += HD + 1)
    unroll_seq(seq, [&](auto sc) __attribute__((always_inline)) { step(sc, g + decltype(sc)::value); });
  // the last stages, with their hidden-ring slots still in the same order
  unroll_seq(seq, [&](auto sc) __attribute__((always_inline)) {
    if (g + decltype(sc)::value < total) step(sc, g + decltype(sc)::value);
  });
}

// --------------------------------------------------------------------------------------------
// K1i: LM-head kernel for decode launches of up to 128 rows. Same MFMA chain (C1), fragment order
// and per-tile epilogue as k_lmhead, hence the same bits.
//
// How fast HBM delivers a W stream depends on its order: DMA probes streaming a 311 MB vocab
// segment from 198 CUs, each owning 3 tiles (192 W rows), reach ~6 TB/s when every request takes
// 512 contiguous bytes of 64 rows of one tile, but ~4.8-5.1 TB/s when a stage takes 128 (or 256)
// bytes of all 192 rows at once, which is how k_lmhead_deep stages W. So here a W stage is one
// tile's 64 rows x 256 K (32 KB), and the block cycles through its NT tiles within each 256-K
// chunk: stage g holds chunk g / NT of tile g % NT, and a chunk of the hidden rows serves NT
// consecutive stages. The hidden rows share each CU's memory path with W, and how they are
// fetched matters as much: the same probes slow from 55 to 77 us (128 rows) when the rows come as
// MFMA fragments (16 rows x 64 bytes per load) but only to 66 us as whole 128-byte lines.
//  - NPW producer waves copy W into a ring of NS stages, keep NS-1 in flight and wait, before
//    each stage's barrier, only for their own copy of that stage;
//  - CW compute waves own 16 NBW rows each and all NT tiles' columns. Each loads its rows' next
//    chunk as whole lines into registers a chunk ahead, writes it into its own slice of an LDS
//    buffer after its last read of the current chunk, and reads its hidden fragments from there
//    (a wave's slice is only ever touched by that wave: its LDS accesses complete in order, so
//    no barrier guards it). The compute waves' loads never wait on W (separate counts).
// One item (NT consecutive tiles of a segment; past a segment's end the rows are clamped and the
// epilogue skips the missing tiles) per block.
// --------------------------------------------------------------------------------------------
template <int CW, int NBW, int NS, int NPW, int NT, bool ENT, bool TEMP, bool PORT>
__global__ void __launch_bounds__(64 * (CW + NPW)) k_lmhead_il(const LmheadArgs a) {
  constexpr int SK = 256;                 // K of a stage and of a hidden chunk
  constexpr int RB = 2 * SK;              // bytes of one staged row (512)
  constexpr int SW = kVocabTile * RB;     // bytes of one W stage (32 KB)
  constexpr int DPS = SW / 1024;          // DMA instructions per stage (1 KB each)
  constexpr int DPW = DPS / NPW;          // ... per producer wave
  constexpr int KS = SK / 32;             // MFMA K-steps per stage
  constexpr int RPI = 1024 / RB;          // staged rows per DMA instruction
  constexpr int BT = 16 * NBW * CW;       // rows of the block
  constexpr int NL = 8 * NBW;             // line loads per compute wave per chunk (1 KB each)
  static_assert(NPW * DPW == DPS && NS >= 3 && (NS - 2) * DPW <= 63 && NT >= 1, "stages");
  static_assert(NS * SW + BT * RB <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t lds_w[NS * SW];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_h[BT * RB];
  // in both buffers, piece c (16 bytes) of staged row r sits at position c ^ (r & 15): a fragment
  // read (16 consecutive rows, one piece each) covers the 64 banks evenly

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int H = a.H;
  const int nc = H / SK;      // K chunks (the launcher checks that SK divides H)
  const int total = nc * NT;  // stages of the block
  Tile t;
  {
    const int ips = (a.tiles_per_seg + NT - 1) / NT;  // items per segment
    const int it = (int)blockIdx.x;
    const int seg = a.seg_begin + it / ips;
    const int jt = (it % ips) * NT;
    const int64_t col0 = (int64_t)jt * kVocabTile;
    t.start = uni64((int64_t)seg * a.seg_len + col0);
    t.len = uni((int)min((int64_t)NT * kVocabTile, a.seg_len - col0));
    t.tile0 = uni(seg * a.tiles_per_seg + jt);
    t.row0 = 0;
    t.rows = a.rows;
  }

  if (wave >= CW) {
    // ---- producer: stage g = (chunk g / NT, tile g % NT) into the ring ----
    const int p = wave - CW;
    const uint32_t lbase = (uint32_t)(uintptr_t)lds_w;
    const i32x4 desc = buffer_desc(a.W + (t.start - a.w_row0) * (int64_t)H, (uint32_t)(t.len * H * 2));
    int rq[DPW], cq[DPW];  // tile row and logical piece of this lane's 16 bytes, per instruction
#pragma unroll
    for (int d = 0; d < DPW; ++d) {
      const int q = d * NPW + p;  // instruction q fills tile rows RPI q .. RPI q + RPI - 1
      rq[d] = RPI * q + lane / (RB / 16);
      cq[d] = (lane % (RB / 16)) ^ (rq[d] & 15);
    }
    auto issue = [&](int g) {
      const int kc = g / NT, u = g % NT;
      const uint32_t dst = (uint32_t)uni((int)(lbase + (uint32_t)(g % NS) * SW));
      const uint32_t so = (uint32_t)uni(kc * RB);
#pragma unroll
      for (int d = 0; d < DPW; ++d) {
        const int r = min(kVocabTile * u + rq[d], t.len - 1);
        dma16_asm(desc, dst + (uint32_t)(d * NPW + p) * 1024u, (uint32_t)(r * H + cq[d] * 8) * 2u, so);
      }
    };
    const int pro = min(NS - 1, total);
    for (int g = 0; g < pro; ++g) issue(g);
    for (int g = 0; g < total; ++g) {
      // stage g has landed (for this wave) once at most the younger stages are in flight
      wait_vm_n<DPW, NS - 2>(min(NS - 2, total - 1 - g));
      __asm__ volatile("s_barrier" ::: "memory");
      // the slot of stage g - 1 is free: every compute wave finished it before this barrier
      if (g + NS - 1 < total) issue(g + NS - 1);
    }
    return;
  }

  // ---- compute waves ----
  const int rows = a.rows;
  const bool has_rows = 16 * NBW * wave < rows;  // uniform: this wave owns a row of the launch
  const int r0 = 16 * NBW * wave;                // the wave's first row (of the launch and of lds_h)
  // Line load i of a chunk: rows 8 (i / 4) .. +7 of the wave (lane >> 3 picks the row, clamped
  // into the launch), bytes 128 (i % 4) + 16 (lane & 7) of the chunk's 512; it lands in lds_h at
  // the row's position for logical piece 8 (i % 4) + (lane & 7), i.e. 16 B unit
  // ((lane & 7) ^ (lane >> 3)) + 8 ((i % 4) ^ ((i / 4) & 1)) of the row (r & 15 = 8 ((i / 4) & 1)
  // + (lane >> 3)).
  const uint8_t* hbase = (const uint8_t*)a.hidden;
  uint32_t goff[2 * NBW];  // per 8-row group
  uint32_t soff[2 * NBW];
#pragma unroll
  for (int q = 0; q < 2 * NBW; ++q) {
    const int lr = r0 + 8 * q + (lane >> 3);
    goff[q] = (uint32_t)(min(lr, rows - 1) * H) * 2u + 16u * (lane & 7);
    soff[q] = (uint32_t)lr * RB + (uint32_t)(((lane & 7) ^ (lane >> 3)) << 4);
  }
  u32x4 hv[NL];
  auto load_lines = [&](int kc) __attribute__((always_inline)) {  // chunk kc (mod nc)
    const uint32_t ko = (uint32_t)(kc % nc) * RB;
#pragma unroll
    for (int i = 0; i < NL; ++i)
      hv[i] = *(const u32x4*)(hbase + goff[i / 4] + ko + 128u * (i % 4));
  };
  auto store_lines = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NL; ++i)
      *(u32x4*)(lds_h + soff[i / 4] + 128u * ((i % 4) ^ ((i / 4) & 1))) = hv[i];
  };
  load_lines(0);
  store_lines();
  load_lines(1);
  const int r16 = lane & 15;
  int loff[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) loff[s] = r16 * RB + (((4 * s + (lane >> 4)) ^ r16) << 4);
  const uint8_t* hp = lds_h + r0 * RB;  // the wave's rows
  f32x4 acc[4 * NT][NBW];
#pragma unroll
  for (int i = 0; i < 4 * NT; ++i)
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.0f;
  int ytgt[NBW];
  load_targets<NBW>(ytgt, a, t, wave, lane);

  int g = 0;
  for (int kc = 0; kc < nc; ++kc) {
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      // every LDS read of the previous stage is done before its slot is handed back
      __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      const uint8_t* sp = lds_w + (g % NS) * SW;
      // W and hidden fragments one K-step ahead of the MFMAs that use them (a wave without rows
      // of the launch computes on clamped rows; only its epilogue is skipped)
      bf16x8 fa[2][4], fb[2][NBW];
      auto frags = [&](int s, int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[slot][i] = *(const bf16x8*)(sp + i * 16 * RB + loff[s]);
#pragma unroll
        for (int j = 0; j < NBW; ++j) fb[slot][j] = *(const bf16x8*)(hp + j * 16 * RB + loff[s]);
      };
      frags(0, 0);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        if (s + 1 < KS) frags(s + 1, (s + 1) & 1);
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[4 * u + i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                fa[s & 1][i], fb[s & 1][j], acc[4 * u + i][j], 0, 0, 0);
      }
      if (u == NT - 1) {
        // after the chunk's last reads of the wave's rows: the next chunk replaces them, and
        // the one after that is fetched (past the last chunk: the first ones again, harmless)
        store_lines();
        load_lines(kc + 2);
      }
      ++g;
    }
  }
  if (has_rows) tile_epilogue<4 * NT, NBW, ENT, TEMP, PORT>(acc, ytgt, a, t, 0, wave, lane);
}

// --------------------------------------------------------------------------------------------
// K2a: fold of one segment's tile partials for 64 rows (C8). Lane = row, so every load of a wave
// is one contiguous 256-byte piece of a [tile][row] array. The block's 16 waves first take the
// segment's tiles round-robin for the exact maximum, then its groups of 32 tiles round-robin,
// each group one sequential chain; wave 0 then runs the pairwise tree over the groups in LDS.
// Each wave issues all loads of a pass (up to UM maxima, a whole group) before it uses them, so a
// pass costs one memory latency rather than one per few tiles.
// With a.done set, the fold of the last segment to finish for a row block also runs the
// cross-segment merge (C9, C10) of those rows, so a forward needs no separate merge launch:
// every block publishes its records, counts itself in done[row block], and the block that
// completes the count reads all records back and writes the outputs.
// --------------------------------------------------------------------------------------------
constexpr int kFoldWaves = 16;

template <int NS, bool ENT, bool PORT>
__device__ __forceinline__ void merge_row(const MergeArgs& a, int t, int32_t y);
template <bool ENT, bool PORT>
__device__ __forceinline__ void merge_one(const MergeArgs& a, int t);

template <bool ENT, bool PORT>
__global__ void __launch_bounds__(64 * kFoldWaves) k_segment_fold(const FoldArgs a) {
  constexpr int G = kFoldGroup;
  constexpr int UM = 40;  // maxima loaded per wave and pass
  __shared__ float red[kFoldWaves][64];
  __shared__ float ga[kMaxFoldGroups][64];
  __shared__ float gb[ENT ? kMaxFoldGroups : 1][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = blockIdx.x * 64 + lane;
  const bool live = t < a.rows;
  const int sl = blockIdx.y;  // segment inside this launch's range
  const int seg = a.seg_begin + sl;
  const int64_t g0 = (int64_t)seg * a.tiles_per_seg - a.g_base;
  const int64_t tc = live ? t : 0;  // dead lanes read row 0 (in bounds) and write nothing
  const float* __restrict__ pm = a.part_m + g0 * a.ld + tc;
  const float* __restrict__ ps = a.part_s + g0 * a.ld + tc;
  const float* __restrict__ pu = ENT ? a.part_u + g0 * a.ld + tc : nullptr;
  const int n = a.tiles_per_seg;
  const int Q = (n + G - 1) / G;

  float M = -INFINITY;
  for (int j0 = wave; j0 < n; j0 += UM * kFoldWaves) {
    float v[UM];
#pragma unroll
    for (int u = 0; u < UM; ++u) {
      const int j = j0 + u * kFoldWaves;
      v[u] = j < n ? pm[(int64_t)j * a.ld] : -INFINITY;
    }
#pragma unroll
    for (int u = 0; u < UM; ++u) M = fmaxf(M, v[u]);
  }
  red[wave][lane] = M;
  __syncthreads();
  M = red[0][lane];
#pragma unroll
  for (int w = 1; w < kFoldWaves; ++w) M = fmaxf(M, red[w][lane]);

  for (int q = wave; q < Q; q += kFoldWaves) {
    const int j0 = q * G;
    const int len = min(n - j0, G);
    float vm[G], vs[G], vu[ENT ? G : 1];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const bool in = u < len;
      const int64_t o = (int64_t)(j0 + u) * a.ld;
      vm[u] = in ? pm[o] : 0.0f;
      vs[u] = in ? ps[o] : 0.0f;
      if constexpr (ENT) vu[u] = in ? pu[o] : 0.0f;
    }
    float A = 0.0f, B = 0.0f;
#pragma unroll
    for (int u = 0; u < G; ++u) {
      if (u < len) {
        const float dm = vm[u] - M;
        const float e = EXP<PORT>(dm);
        A = A + vs[u] * e;
        if constexpr (ENT) B = B + (vu[u] + vs[u] * dm) * e;
      }
    }
    ga[q][lane] = A;
    if constexpr (ENT) gb[q][lane] = B;
  }
  __syncthreads();
  if (wave != 0) return;
  // pairwise tree over the groups in index order; a missing right member passes the left through
  for (int st = 1; st < Q; st *= 2) {
    for (int q = 0; q + st < Q; q += 2 * st) {
      ga[q][lane] = ga[q][lane] + ga[q + st][lane];
      if constexpr (ENT) gb[q][lane] = gb[q][lane] + gb[q + st][lane];
    }
  }
  if (live) {
    const int32_t y = a.targets[t];
    const int64_t lo = (int64_t)seg * a.seg_len;
    const bool owner = y >= 0 && (int64_t)y >= lo && (int64_t)y < lo + a.seg_len;
    rlk_segment_record_t r;
    r.m = M;
    r.s = ga[0][lane];
    r.u = ENT ? gb[0][lane] : 0.0f;
    r.tgt = owner ? a.tgt[t] : __builtin_nanf("");
    a.rec[(int64_t)sl * a.rec_ld + t] = r;
  }
  if (a.done == nullptr) return;
  // publish this segment's records device-wide, then count it for the row block
  __threadfence();
  uint32_t prev = 0;
  if (lane == 0)
    prev = __hip_atomic_fetch_add(a.done + blockIdx.x, 1u, __ATOMIC_ACQ_REL,
                                  __HIP_MEMORY_SCOPE_AGENT);
  prev = (uint32_t)__builtin_amdgcn_readfirstlane((int)prev);
  if (prev != (uint32_t)gridDim.y - 1) return;
  // the last segment of this row block: every other block's records are visible now
  __threadfence();
  if (lane == 0) __hip_atomic_store(a.done + blockIdx.x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (live) merge_one<ENT, PORT>(a.mg, t);
}

// --------------------------------------------------------------------------------------------
// K2b: per row cross-segment merge and outputs (C9, C10).
// --------------------------------------------------------------------------------------------
template <int NS, bool ENT, bool PORT>
__device__ __forceinline__ void merge_row(const MergeArgs& a, int t, int32_t y) {
  float Ms[NS], Ss[NS], Us[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const rlk_segment_record_t r = a.rec[(int64_t)s * a.rec_ld + t];
    Ms[s] = r.m;
    Ss[s] = r.s;
    Us[s] = r.u;
  }
  float M = Ms[0];
#pragma unroll
  for (int s = 1; s < NS; ++s) M = fmaxf(M, Ms[s]);
  float as[NS], au[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const float dm = Ms[s] - M;
    const float e = EXP<PORT>(dm);
    as[s] = Ss[s] * e;
    if constexpr (ENT) au[s] = (Us[s] + Ss[s] * dm) * e;
  }
  const float S = tree_sum<NS>(as);
  const float logS = LOG<PORT>(S);
  const float lse = M + logS;
  const int owner = (int)((int64_t)y / a.seg_len);
  const float zy = a.rec[(int64_t)owner * a.rec_ld + t].tgt;
  a.logp[t] = zy - lse;
  a.lse[t] = lse;
  if constexpr (ENT) {
    const float U = tree_sum<NS>(au);
    a.entropy[t] = logS - U / S;
  }
}

// Outputs of row t (C10), including padded rows and out-of-range targets.
template <bool ENT, bool PORT>
__device__ __forceinline__ void merge_one(const MergeArgs& a, int t) {
  const int32_t y = a.targets[t];
  if (y < 0) {
    a.logp[t] = 0.0f;
    a.lse[t] = 0.0f;
    if constexpr (ENT) a.entropy[t] = 0.0f;
    return;
  }
  if ((int64_t)y >= a.vocab) {
    const float nan = __builtin_nanf("");
    a.logp[t] = nan;
    a.lse[t] = nan;
    if constexpr (ENT) a.entropy[t] = nan;
    if (a.status) atomicOr(a.status, (unsigned)RLK_DEVICE_STATUS_BAD_TARGET);
    return;
  }
  switch (a.n_seg) {
    case 1: merge_row<1, ENT, PORT>(a, t, y); break;
    case 2: merge_row<2, ENT, PORT>(a, t, y); break;
    case 4: merge_row<4, ENT, PORT>(a, t, y); break;
    default: merge_row<8, ENT, PORT>(a, t, y); break;
  }
}

template <bool ENT, bool PORT>
__global__ void __launch_bounds__(256) k_merge(const MergeArgs a) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= a.rows) return;
  merge_one<ENT, PORT>(a, t);
}

// --------------------------------------------------------------------------------------------
// K0: final RMSNorm, one 64-wide wave per row (C12).
// --------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_rmsnorm(const RmsArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const uint16_t* __restrict__ x = a.x + (int64_t)row * a.H;
  uint16_t* __restrict__ y = a.y + (int64_t)row * a.H;
  const int npieces = a.H / 8;
  float ss = 0.0f;
  for (int p = lane; p < npieces; p += 64) {
    const u32x4 v = *(const u32x4*)(x + p * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float lo = bf16_to_f32(v[w] & 0xffffu);
      const float hi = bf16_to_f32(v[w] >> 16);
      ss = ss + lo * lo;
      ss = ss + hi * hi;
    }
  }
  ss = ss + __shfl_xor(ss, 32);
  ss = ss + __shfl_xor(ss, 16);
  ss = ss + __shfl_xor(ss, 8);
  ss = ss + __shfl_xor(ss, 4);
  ss = ss + __shfl_xor(ss, 2);
  ss = ss + __shfl_xor(ss, 1);
  const float v = ss * a.inv_H + a.eps;
  const float r = a.portable ? p_rsq(v) : c_rsq(v);
  for (int p = lane; p < npieces; p += 64) {
    const u32x4 v = *(const u32x4*)(x + p * 8);
    const u32x4 g = *(const u32x4*)(a.gamma + p * 8);
    u32x4 o;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float lo = (bf16_to_f32(v[w] & 0xffffu) * r) * bf16_to_f32(g[w] & 0xffffu);
      const float hi = (bf16_to_f32(v[w] >> 16) * r) * bf16_to_f32(g[w] >> 16);
      o[w] = (uint32_t)bf16_rne(lo) | ((uint32_t)bf16_rne(hi) << 16);
    }
    *(u32x4*)(y + p * 8) = o;
  }
}

// Clears the status word and the LM-head work queues that follow it in its 128-byte slot, and
// the fused-merge counters of the segment fold.
__global__ void k_clear_status(uint32_t* status, uint32_t* done, int64_t n_done) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < kStatusSlotWords) status[i] = 0u;
  if (done && i < n_done) done[i] = 0u;
}

// --------------------------------------------------------------------------------------------
// launchers
// --------------------------------------------------------------------------------------------
bool token_tile_supported(int bt) { return bt == 32 || bt == 64 || bt == 128 || bt == 256; }

// Blocks of a launch: per band of row tiles, vocab blocks of NTPB tiles per segment x the band's
// row tiles, rounded up to a multiple of 8 (the XCD remap in map_tile; extra blocks exit at once).
template <int BT, int NTPB>
static int64_t lmhead_blocks(const LmheadArgs& a) {
  const int64_t n_vb = (int64_t)a.n_seg * ((a.tiles_per_seg + NTPB - 1) / NTPB);
  const int64_t n_tt = (a.rows + BT - 1) / BT;
  if (n_vb == 0 || n_tt == 0) return 0;
  const int64_t rb = band_row_tiles<BT>(a.H);
  const int64_t n_full = n_tt / rb, rest = n_tt - n_full * rb;
  return n_full * band_blocks(n_vb, rb) + (rest ? band_blocks(n_vb, rest) : 0);
}

// Calls f with the entropy, temperature and portable-primitive modes of a launch as compile-time
// constants, so each kernel instance carries only the epilogue it runs.
template <class F>
static void with_modes(const LmheadArgs& a, bool ent, F&& f) {
  using T = std::true_type;
  using N = std::false_type;
  const bool temp = a.inv_tau != 1.0f;
  if (a.portable) {
    if (ent) temp ? f(T{}, T{}, T{}) : f(T{}, N{}, T{});
    else temp ? f(N{}, T{}, T{}) : f(N{}, N{}, T{});
  } else {
    if (ent) temp ? f(T{}, T{}, N{}) : f(T{}, N{}, N{});
    else temp ? f(N{}, T{}, N{}) : f(N{}, N{}, N{});
  }
}

// Persistent launch: one block per CU (the kernel's LDS allows no second), fewer when there are
// fewer items; the queues must be zero (k_clear_status), and the kernel leaves them zero.
template <int VW, int TW, int NTB>
static hipError_t launch_variant(const LmheadArgs& a, bool ent, hipStream_t s) {
  constexpr int BT = 32 * NTB * TW;
  const int64_t n_vb = (int64_t)a.n_seg * ((a.tiles_per_seg + 3) / 4);
  const int64_t n_tt = (a.rows + BT - 1) / BT;
  const int64_t items = n_vb * n_tt;
  if (items == 0) return hipSuccess;
  if (!a.queue || items > 0x7fffffffLL - 8 * 4096) return hipErrorInvalidValue;
  LmheadArgs q = a;
  queue_setup(q, n_vb, n_tt, band_row_tiles<BT>(a.H));
  const int64_t blocks = std::min<int64_t>(items, a.n_cu > 0 ? a.n_cu : 256);
  const dim3 grid((unsigned)blocks), block(64 * VW * TW);
  with_modes(a, ent, [&](auto e, auto t, auto p) {
    hipLaunchKernelGGL((k_lmhead<VW, TW, NTB, e.value, t.value, p.value>), grid, block, 0, s, q);
  });
  return hipGetLastError();
}

template <int CW, int NBW, int HD, int SK, int NS, int NPW>
static hipError_t launch_stream(const LmheadArgs& a, bool ent, hipStream_t s) {
  const int64_t items = (int64_t)a.n_seg * a.tiles_per_seg;
  if (items == 0 || a.rows == 0) return hipSuccess;
  if (a.rows > 16 * NBW * CW) return hipErrorInvalidValue;  // every row needs a compute wave
  // as few blocks as give every block the same number of items (+-1) at the least items per
  // block: 594 tiles on 256 CUs -> 198 blocks of 3 (not 82 of 3 and 174 of 2)
  const int64_t cu = a.n_cu > 0 ? a.n_cu : 256;
  const int64_t per = (items + cu - 1) / cu;
  const int64_t blocks = (items + per - 1) / per;
  const dim3 grid((unsigned)blocks), block(64 * (CW + NPW));
  with_modes(a, ent, [&](auto e, auto t, auto p) {
    hipLaunchKernelGGL((k_lmhead_stream<CW, NBW, SK, NS, NPW, HD, e.value, t.value, p.value>), grid,
                       block, 0, s, a);
  });
  return hipGetLastError();
}

template <int CW, int NBW, int NS, int NPW, int NT>
static hipError_t launch_il(const LmheadArgs& a, bool ent, hipStream_t s) {
  const int64_t items = (int64_t)a.n_seg * ((a.tiles_per_seg + NT - 1) / NT);
  if (items == 0 || a.rows == 0) return hipSuccess;
  if (a.rows > 16 * NBW * CW || a.H % 256 != 0) return hipErrorInvalidValue;
  if (items > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)items), block(64 * (CW + NPW));
  with_modes(a, ent, [&](auto e, auto t, auto p) {
    hipLaunchKernelGGL((k_lmhead_il<CW, NBW, NS, NPW, NT, e.value, t.value, p.value>), grid, block,
                       0, s, a);
  });
  return hipGetLastError();
}

template <int VW, int TW, int NB16, int NS, int NTPB, int HS = 0>
static hipError_t launch_deep(const LmheadArgs& a, bool ent, hipStream_t s) {
  constexpr int BT = 16 * NB16 * TW;
  const int64_t blocks = lmhead_blocks<BT, NTPB>(a);
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks), block(64 * VW * TW);
  with_modes(a, ent, [&](auto e, auto t, auto p) {
    hipLaunchKernelGGL((k_lmhead_deep<VW, TW, NB16, NS, NTPB, HS, e.value, t.value, p.value>), grid,
                       block, 0, s, a);
  });
  return hipGetLastError();
}

// Launch shape for token_tile 0 (every choice gives the same bits). Launches past 256 rows take
// the 256-row tile of k_lmhead. Up to 256 rows (decode batches) there is one row tile, and the
// launch is bound by how many columns its busiest CU streams and multiplies: blocks of 3 tiles
// (192 columns) spread a Qwen3-8B vocab segment over 198 blocks instead of 149, so they are taken
// whenever they put fewer columns on the busiest CU than blocks of 4 tiles do, with row tiles of
// 64 to 256 rows (never more than 63 rows of padding). token_tile 32/64/128/256 forces blocks of
// 4 tiles with that row tile.
static bool three_tile_blocks(const LmheadArgs& a) {
  const int64_t cu = a.n_cu > 0 ? a.n_cu : 256;
  const int64_t n3 = (int64_t)a.n_seg * ((a.tiles_per_seg + 2) / 3);
  const int64_t n4 = (int64_t)a.n_seg * ((a.tiles_per_seg + 3) / 4);
  return (n3 + cu - 1) / cu * 3 < (n4 + cu - 1) / cu * 4;
}

hipError_t launch_lmhead(const LmheadArgs& a, int bt, bool ent, hipStream_t s) {
  if (bt == 0) {
    if (a.rows > 256) return launch_variant<2, 4, 2>(a, ent, s);
    // up to 128 rows: W streamed tile by tile in 512-byte rows, the hidden rows fetched as
    // whole lines (k_lmhead_il; per 311 MB vocab segment 59-61 us up to 64 rows and 66-68 us up
    // to 128, against 64-72 us for the streaming kernel and 3-tile blocks); up to 16 rows the
    // streaming kernel
    if (a.rows <= 128 && a.H % 256 == 0) {
      if (a.rows <= 16) return launch_stream<1, 1, 2, 256, 4, 4>(a, ent, s);
      if (a.rows <= 32) return launch_il<2, 1, 4, 4, 3>(a, ent, s);
      if (a.rows <= 64) return launch_il<4, 1, 4, 4, 3>(a, ent, s);
      return launch_il<8, 1, 3, 4, 3>(a, ent, s);
    }
    if (a.rows <= 32) return launch_stream<2, 1, 3, 128, 8, 2>(a, ent, s);
    if (three_tile_blocks(a)) {
      if (a.rows > 192) return launch_deep<3, 4, 4, 3, 3, 2>(a, ent, s);
      // 12 waves (3 per SIMD; 6 waves would load two SIMDs with two waves and two with one):
      // 48, 32 or 16 rows per wave, W and the hidden rows in one ring of 3 (4) stages
      if (a.rows > 128) return launch_deep<3, 4, 3, 3, 3>(a, ent, s);
      if (a.rows > 64) return launch_deep<3, 4, 2, 3, 3>(a, ent, s);
      return launch_deep<3, 4, 1, 4, 3>(a, ent, s);
    }
    bt = a.rows > 128 ? 256 : a.rows > 64 ? 128 : a.rows > 32 ? 64 : 32;
  }
  switch (bt) {
    case 256: return launch_variant<2, 4, 2>(a, ent, s);
    case 128: return launch_deep<2, 2, 4, 3, 4>(a, ent, s);
    case 64: return launch_deep<4, 1, 4, 3, 4>(a, ent, s);
    case 32: return launch_deep<4, 1, 2, 4, 4>(a, ent, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fold(const FoldArgs& a, bool ent, hipStream_t s) {
  if (a.rows == 0 || a.n_seg == 0) return hipSuccess;
  if ((a.tiles_per_seg + kFoldGroup - 1) / kFoldGroup > kMaxFoldGroups) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((a.rows + 63) / 64), (unsigned)a.n_seg), block(64 * kFoldWaves);
  if (a.portable) {
    if (ent) hipLaunchKernelGGL((k_segment_fold<true, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_segment_fold<false, true>), grid, block, 0, s, a);
  } else {
    if (ent) hipLaunchKernelGGL((k_segment_fold<true, false>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_segment_fold<false, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, bool ent, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  const dim3 grid((unsigned)((a.rows + 255) / 256)), block(256);
  if (a.portable) {
    if (ent) hipLaunchKernelGGL((k_merge<true, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_merge<false, true>), grid, block, 0, s, a);
  } else {
    if (ent) hipLaunchKernelGGL((k_merge<true, false>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_merge<false, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const RmsArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  const dim3 grid((unsigned)((a.rows + 3) / 4)), block(256);
  hipLaunchKernelGGL(k_rmsnorm, grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_clear_status(uint32_t* status, uint32_t* done, int64_t n_done, hipStream_t s) {
  const int64_t n = std::max<int64_t>(kStatusSlotWords, done ? n_done : 0);
  hipLaunchKernelGGL(k_clear_status, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, status,
                     done, n_done);
  return hipGetLastError();
}

}  // namespace rlk
