// Host side of the C ABI: validation, layout planning, workspace carving and launches.
//
// Strict mode only: every unsupported case returns an error naming why and enqueues nothing;
// there is no fallback path (RL-Kernel v0.1.0 summary page, "Numeric execution contract": a
// strict path either runs the declared contract or reports that it cannot). The layout
// descriptor only changes which launches are made — the per-row arithmetic is the kernels'
// (the aihirek.info report, "A vime és az RL-Kernel eltérő feladatot kapott": memory layouts and
// schedules may differ as long as they do not change the numerics being compared).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "rlk_internal.h"
#include "rlk_logprob.h"

#ifndef RLK_BUILD_FLAGS
#define RLK_BUILD_FLAGS "unknown"
#endif

#define RLK_API extern "C" __attribute__((visibility("default")))

struct rlk_logprob {
  rlk_logprob_config_t cfg;
  int device;
  int n_cu;  // compute units of the device
  std::string contract;
  void* scratch;  // device address of this device's scratch array (allocation-free forward)
};

// The workspace of rlk_logprob_forward_noalloc: a fixed array in device memory, one copy per GPU
// the library is loaded on, held until the process ends. In host code its name is only a
// stand-in, never a device address: the address is resolved with hipGetSymbolAddress, once per
// device, with that device current, and only that address is handed to kernels.
constexpr size_t kScratchBytes = (size_t)64 << 20;  // RLK_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == RLK_NOALLOC_SCRATCH_BYTES, "header and library agree");
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

thread_local std::string g_last_error;

rlk_status_t fail(rlk_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

rlk_status_t ok() {
  g_last_error.clear();
  return RLK_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Geometry {
  int64_t seg_len;
  int32_t tiles_per_seg;
  int32_t n_tiles;
};

Geometry geometry(const rlk_logprob_config_t& c) {
  Geometry g;
  g.seg_len = c.vocab_size / c.vocab_segments;
  g.tiles_per_seg = (int32_t)((g.seg_len + rlk::kVocabTile - 1) / rlk::kVocabTile);
  g.n_tiles = g.tiles_per_seg * c.vocab_segments;
  return g;
}

rlk_status_t check_config(const rlk_logprob_config_t* c) {
  if (!c) return fail(RLK_ERR_INVALID_ARGUMENT, "config is NULL");
  if (c->reserved != 0) return fail(RLK_ERR_INVALID_ARGUMENT, "config.reserved must be 0");
  if (c->flags & ~(RLK_FLAG_RMSNORM | RLK_FLAG_ENTROPY | RLK_FLAG_PORTABLE_EXP))
    return fail(RLK_ERR_INVALID_ARGUMENT, "unknown flag bits 0x%x", c->flags);
  if (c->hidden_size <= 0 || c->hidden_size % 128 != 0 || c->hidden_size > 65536)
    return fail(RLK_ERR_UNSUPPORTED_SHAPE, "hidden_size %d is not a positive multiple of 128 <= 65536",
                c->hidden_size);
  const int s = c->vocab_segments;
  if (s != 1 && s != 2 && s != 4 && s != 8)
    return fail(RLK_ERR_UNSUPPORTED_SHAPE, "vocab_segments %d is not 1, 2, 4 or 8", s);
  if (c->vocab_size <= 0 || c->vocab_size % s != 0)
    return fail(RLK_ERR_UNSUPPORTED_SHAPE, "vocab_size %lld is not a positive multiple of %d",
                (long long)c->vocab_size, s);
  constexpr int64_t kMaxSegLen = (int64_t)rlk::kMaxFoldGroups * rlk::kFoldGroup * rlk::kVocabTile;
  if (c->vocab_size / s > kMaxSegLen)
    return fail(RLK_ERR_UNSUPPORTED_SHAPE, "vocab segment of %lld columns is longer than %lld",
                (long long)(c->vocab_size / s), (long long)kMaxSegLen);
  if (c->vocab_size > 0x7fffffffLL)
    return fail(RLK_ERR_UNSUPPORTED_SHAPE, "vocab_size does not fit int32 targets");
  if (!std::isfinite(c->inv_temperature) || !(c->inv_temperature > 0.0f))
    return fail(RLK_ERR_INVALID_ARGUMENT, "inv_temperature must be finite and > 0");
  if ((c->flags & RLK_FLAG_RMSNORM) && !(std::isfinite(c->rms_eps) && c->rms_eps >= 0.0f))
    return fail(RLK_ERR_INVALID_ARGUMENT, "rms_eps must be finite and >= 0");
  return RLK_OK;
}

struct RowRange {
  int64_t begin, end;
};

// One LM-head launch group: a row range (of one batch chunk) x one vocab shard.
struct Plan {
  std::vector<RowRange> batches;          // merge granularity
  std::vector<std::vector<RowRange>> chunks;  // per batch
  int32_t shards;
  int64_t launches;
};

rlk_status_t plan_layout(const rlk_logprob_config_t& c, const rlk_layout_desc_t* l, Plan* p) {
  if (!l) return fail(RLK_ERR_INVALID_ARGUMENT, "layout is NULL");
  if (l->reserved != 0) return fail(RLK_ERR_INVALID_ARGUMENT, "layout.reserved must be 0");
  if (l->num_rows < 0 || l->num_rows > 0x7fffffffLL)
    return fail(RLK_ERR_INVALID_ARGUMENT, "num_rows %lld out of range", (long long)l->num_rows);
  if (l->row_chunk < 0) return fail(RLK_ERR_INVALID_ARGUMENT, "row_chunk < 0");
  if (l->token_tile != 0 && !rlk::token_tile_supported(l->token_tile))
    return fail(RLK_ERR_UNSUPPORTED_SHAPE, "token_tile %d is not 0, 32, 64, 128 or 256", l->token_tile);
  const int32_t ns = l->vocab_shards == 0 ? 1 : l->vocab_shards;
  if (ns < 1 || ns > c.vocab_segments || c.vocab_segments % ns != 0)
    return fail(RLK_ERR_CONTRACT, "vocab_shards %d does not divide vocab_segments %d", ns,
                c.vocab_segments);
  const int64_t T = l->num_rows;
  p->batches.clear();
  p->chunks.clear();
  if (l->num_batches <= 1) {
    if (l->num_batches == 1 && l->batch_offsets &&
        (l->batch_offsets[0] != 0 || l->batch_offsets[1] != T))
      return fail(RLK_ERR_INVALID_ARGUMENT, "single batch offsets must be [0, num_rows]");
    if (l->num_batches < 0) return fail(RLK_ERR_INVALID_ARGUMENT, "num_batches < 0");
    p->batches.push_back({0, T});
  } else {
    const int64_t* o = l->batch_offsets;
    if (!o) return fail(RLK_ERR_INVALID_ARGUMENT, "num_batches > 1 needs batch_offsets");
    if (o[0] != 0 || o[l->num_batches] != T)
      return fail(RLK_ERR_INVALID_ARGUMENT, "batch_offsets must start at 0 and end at num_rows");
    for (int32_t b = 0; b < l->num_batches; ++b) {
      if (o[b + 1] < o[b]) return fail(RLK_ERR_INVALID_ARGUMENT, "batch_offsets not ascending");
      p->batches.push_back({o[b], o[b + 1]});
    }
  }
  p->shards = ns;
  p->launches = 0;
  for (const RowRange& b : p->batches) {
    std::vector<RowRange> ch;
    const int64_t n = b.end - b.begin;
    const int64_t step = l->row_chunk > 0 ? l->row_chunk : std::max<int64_t>(n, 1);
    for (int64_t r = b.begin; r < b.end; r += step) ch.push_back({r, std::min(b.end, r + step)});
    p->launches += (int64_t)ch.size() * ns;
    p->chunks.push_back(std::move(ch));
  }
  return RLK_OK;
}

// Workspace map (offsets in bytes, each 256-aligned).
struct WsMap {
  size_t status, tgt, pm, ps, pu, rec, y, done, total;
};

WsMap ws_map(const rlk_logprob_config_t& c, int64_t rows, int32_t n_tiles, int32_t n_rec_seg) {
  const bool ent = c.flags & RLK_FLAG_ENTROPY;
  const bool rms = c.flags & RLK_FLAG_RMSNORM;
  WsMap m;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = round_up(off + bytes, 256);
    return at;
  };
  const size_t rowsz = (size_t)std::max<int64_t>(rows, 1);
  m.status = take(rlk::kStatusSlotWords * 4);  // status word + LM-head work queues
  m.tgt = take(rowsz * 4);
  m.pm = take((size_t)n_tiles * rowsz * 4);
  m.ps = take((size_t)n_tiles * rowsz * 4);
  m.pu = ent ? take((size_t)n_tiles * rowsz * 4) : 0;
  m.rec = n_rec_seg ? take((size_t)n_rec_seg * rowsz * sizeof(rlk_segment_record_t)) : 0;
  m.y = rms ? take(rowsz * (size_t)c.hidden_size * 2) : 0;
  m.done = n_rec_seg ? take((rowsz + 63) / 64 * 4) : 0;  // fused-merge counters per 64 rows
  m.total = off;
  return m;
}

struct DeviceGuard {
  int prev = -1;
  bool changed = false;
  hipError_t err = hipSuccess;
  explicit DeviceGuard(int dev) {
    err = hipGetDevice(&prev);
    if (err == hipSuccess && prev != dev) {
      err = hipSetDevice(dev);
      changed = err == hipSuccess;
    }
  }
  ~DeviceGuard() {
    if (changed) (void)hipSetDevice(prev);
  }
};

rlk_status_t hip_fail(hipError_t e, const char* what) {
  return fail(RLK_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];  // per device, resolved once

// The device address of `device`'s scratch array; the device must be current.
rlk_status_t resolve_scratch(int device, void** out) {
  *out = nullptr;
  if (device < 0 || device >= kMaxScratchDevices)
    return fail(RLK_ERR_NO_DEVICE, "device %d: no scratch slot (at most %d devices)", device,
                kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[device] = p;
  }
  *out = g_scratch_ptr[device];
  return RLK_OK;
}

// RMSNorm (optional) then the LM-head tile kernel over rows [r0, r1) and segments [s0, s1).
rlk_status_t run_rows(const rlk_logprob* h, const Geometry& g, const void* hidden, const void* W,
                      int64_t w_row0, const int32_t* targets, const void* gamma, const WsMap& m,
                      uint8_t* ws, int64_t ld, int32_t g_base, int64_t r0, int64_t r1, int s0,
                      int s1, int token_tile, bool do_norm, hipStream_t st) {
  const rlk_logprob_config_t& c = h->cfg;
  const int64_t n = r1 - r0;
  if (n <= 0) return RLK_OK;
  const uint16_t* hid = static_cast<const uint16_t*>(hidden);
  if (c.flags & RLK_FLAG_RMSNORM) {
    uint16_t* y = reinterpret_cast<uint16_t*>(ws + m.y);
    if (do_norm) {
      rlk::RmsArgs ra;
      ra.x = hid + r0 * (int64_t)c.hidden_size;
      ra.gamma = static_cast<const uint16_t*>(gamma);
      ra.y = y + r0 * (int64_t)c.hidden_size;
      ra.rows = (int32_t)n;
      ra.H = c.hidden_size;
      ra.inv_H = 1.0f / (float)c.hidden_size;
      ra.eps = c.rms_eps;
      ra.portable = (c.flags & RLK_FLAG_PORTABLE_EXP) ? 1 : 0;
      hipError_t e = rlk::launch_rmsnorm(ra, st);
      if (e != hipSuccess) return hip_fail(e, "rmsnorm launch");
    }
    hid = y;
  }
  const bool ent = c.flags & RLK_FLAG_ENTROPY;
  rlk::LmheadArgs a;
  a.hidden = hid + r0 * (int64_t)c.hidden_size;
  a.W = static_cast<const uint16_t*>(W);
  a.targets = targets + r0;
  a.part_m = reinterpret_cast<float*>(ws + m.pm) + r0;
  a.part_s = reinterpret_cast<float*>(ws + m.ps) + r0;
  a.part_u = ent ? reinterpret_cast<float*>(ws + m.pu) + r0 : nullptr;
  a.tgt = reinterpret_cast<float*>(ws + m.tgt) + r0;
  a.ld = ld;
  a.w_row0 = w_row0;
  a.seg_len = g.seg_len;
  a.rows = (int32_t)n;
  a.H = c.hidden_size;
  a.tiles_per_seg = g.tiles_per_seg;
  a.seg_begin = s0;
  a.n_seg = s1 - s0;
  a.g_base = g_base;
  a.n_cu = h->n_cu;
  a.portable = (c.flags & RLK_FLAG_PORTABLE_EXP) ? 1 : 0;
  a.inv_tau = c.inv_temperature;
  a.queue = reinterpret_cast<uint32_t*>(ws + m.status) + rlk::kQueueWord;
  hipError_t e = rlk::launch_lmhead(a, token_tile, ent, st);
  if (e != hipSuccess) return hip_fail(e, "lm-head launch");
  return RLK_OK;
}

}  // namespace

// ============================================================================================
RLK_API const char* rlk_status_string(rlk_status_t s) {
  switch (s) {
    case RLK_OK: return "ok";
    case RLK_ERR_INVALID_ARGUMENT: return "invalid argument";
    case RLK_ERR_NO_DEVICE: return "no HIP device";
    case RLK_ERR_UNSUPPORTED_ARCH: return "unsupported GPU architecture (gfx950 only)";
    case RLK_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
    case RLK_ERR_ALIGNMENT: return "misaligned pointer";
    case RLK_ERR_WORKSPACE: return "workspace missing or too small";
    case RLK_ERR_CONTRACT: return "numeric contract violated";
    case RLK_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

RLK_API const char* rlk_last_error(void) { return g_last_error.c_str(); }

RLK_API const char* rlk_build_fingerprint(void) {
  static const std::string fp = std::string("rlk_logprob contract v") +
                                std::to_string(rlk::kContractVersion) +
                                "; target gfx950; compiler " + __clang_version__ +
                                "; flags " + RLK_BUILD_FLAGS;
  return fp.c_str();
}

RLK_API rlk_status_t rlk_logprob_create(const rlk_logprob_config_t* config, int device,
                                        rlk_logprob_t* out) {
  if (!out) return fail(RLK_ERR_INVALID_ARGUMENT, "out is NULL");
  *out = nullptr;
  rlk_status_t st = check_config(config);
  if (st != RLK_OK) return st;
  int count = 0;
  hipError_t e = hipGetDeviceCount(&count);
  if (e != hipSuccess || count <= 0) return fail(RLK_ERR_NO_DEVICE, "no HIP device visible");
  if (device < 0 || device >= count)
    return fail(RLK_ERR_NO_DEVICE, "device %d does not exist (%d visible)", device, count);
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, device);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(RLK_ERR_UNSUPPORTED_ARCH, "device %d is %s, not gfx950", device, prop.gcnArchName);
  void* scr = nullptr;
  {
    DeviceGuard guard(device);
    if (guard.err != hipSuccess) return hip_fail(guard.err, "hipSetDevice");
    st = resolve_scratch(device, &scr);
    if (st != RLK_OK) return st;
  }
  rlk_logprob* h = new (std::nothrow) rlk_logprob;
  if (!h) return fail(RLK_ERR_INVALID_ARGUMENT, "out of host memory");
  h->cfg = *config;
  h->device = device;
  h->n_cu = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
  h->scratch = scr;
  uint32_t itb;
  std::memcpy(&itb, &config->inv_temperature, 4);
  uint32_t epsb;
  std::memcpy(&epsb, &config->rms_eps, 4);
  const bool port = config->flags & RLK_FLAG_PORTABLE_EXP;
  char buf[640];
  snprintf(buf, sizeof(buf),
           "rlk-logprob/v%d;mfma=v_mfma_f32_16x16x32_bf16;kstep=32;bv=%d;H=%d;V=%lld;Sc=%d;"
           "intile=seq16+pair4;segfold=seq%d+pair;segmerge=pair;%s;inv_tau=0x%08x;rms=%d;"
           "rms_eps=0x%08x;%s;rms_tree=lane-seq8+xor32..1;entropy=%d;contract=off",
           rlk::kContractVersion, rlk::kVocabTile, config->hidden_size,
           (long long)config->vocab_size, config->vocab_segments, rlk::kFoldGroup,
           port ? "exp=soft(cw2+taylor7+scale2^n);log=soft(atanh11+cw2)"
                : "exp=v_exp_f32(x*0x3fb8aa3b);log=v_log_f32*0x3f317218",
           itb, (config->flags & RLK_FLAG_RMSNORM) ? 1 : 0,
           (config->flags & RLK_FLAG_RMSNORM) ? epsb : 0u,
           port ? "rsq=1/sqrt(rn)" : "rsq=v_rsq_f32",
           (config->flags & RLK_FLAG_ENTROPY) ? 1 : 0);
  h->contract = buf;
  *out = h;
  return ok();
}

RLK_API rlk_status_t rlk_logprob_destroy(rlk_logprob_t h) {
  delete h;
  return ok();
}

RLK_API const char* rlk_logprob_contract_id(rlk_logprob_t h) { return h ? h->contract.c_str() : ""; }

RLK_API rlk_status_t rlk_layout_check(const rlk_logprob_config_t* config,
                                      const rlk_layout_desc_t* layout, int64_t* num_launches) {
  rlk_status_t st = check_config(config);
  if (st != RLK_OK) return st;
  Plan p;
  st = plan_layout(*config, layout, &p);
  if (st != RLK_OK) return st;
  if (num_launches) *num_launches = p.launches;
  return ok();
}

RLK_API rlk_status_t rlk_logprob_workspace_size(const rlk_logprob_config_t* config,
                                                const rlk_layout_desc_t* layout, size_t* bytes) {
  if (!bytes) return fail(RLK_ERR_INVALID_ARGUMENT, "bytes is NULL");
  rlk_status_t st = check_config(config);
  if (st != RLK_OK) return st;
  Plan p;
  st = plan_layout(*config, layout, &p);
  if (st != RLK_OK) return st;
  const Geometry g = geometry(*config);
  *bytes = ws_map(*config, layout->num_rows, g.n_tiles, config->vocab_segments).total;
  return ok();
}

namespace {
rlk_status_t forward_impl(rlk_logprob_t h, const void* hidden, const void* W_lm,
                          const int32_t* targets, const rlk_layout_desc_t* layout,
                          const void* rms_gamma, float* logp, float* lse, float* entropy,
                          void* workspace, size_t workspace_bytes, rlk_stream_t stream,
                          void* const* events, int32_t num_events) {
  if (!h) return fail(RLK_ERR_INVALID_ARGUMENT, "handle is NULL");
  const rlk_logprob_config_t& c = h->cfg;
  Plan p;
  rlk_status_t st = plan_layout(c, layout, &p);
  if (st != RLK_OK) return st;
  const int64_t T = layout->num_rows;
  const bool ent = c.flags & RLK_FLAG_ENTROPY;
  const bool rms = c.flags & RLK_FLAG_RMSNORM;
  if (T > 0) {
    if (!hidden || !W_lm || !targets || !logp || !lse)
      return fail(RLK_ERR_INVALID_ARGUMENT, "hidden, W_lm, targets, logp and lse are required");
    if (ent && !entropy) return fail(RLK_ERR_INVALID_ARGUMENT, "entropy output required");
    if (rms && !rms_gamma) return fail(RLK_ERR_INVALID_ARGUMENT, "rms_gamma required");
    if (!aligned16(hidden) || !aligned16(W_lm) || !aligned16(targets) || !aligned16(logp) ||
        !aligned16(lse) || (entropy && !aligned16(entropy)) || (rms_gamma && !aligned16(rms_gamma)))
      return fail(RLK_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
  }
  if (!ent && entropy) return fail(RLK_ERR_CONTRACT, "entropy given but RLK_FLAG_ENTROPY not set");
  if (!rms && rms_gamma) return fail(RLK_ERR_CONTRACT, "rms_gamma given but RLK_FLAG_RMSNORM not set");
  const Geometry g = geometry(c);
  const WsMap m = ws_map(c, T, g.n_tiles, c.vocab_segments);
  if (!workspace || workspace_bytes < m.total)
    return fail(RLK_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", m.total, workspace_bytes);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(RLK_ERR_ALIGNMENT, "workspace must be 256-byte aligned");
  DeviceGuard guard(h->device);
  if (guard.err != hipSuccess) return hip_fail(guard.err, "hipSetDevice");
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint32_t* status = reinterpret_cast<uint32_t*>(ws + m.status);
  uint32_t* done = reinterpret_cast<uint32_t*>(ws + m.done);
  hipError_t e = rlk::launch_clear_status(status, done, (T + 63) / 64, s);
  if (e != hipSuccess) return hip_fail(e, "status clear launch");
  if (T == 0) return ok();

  const int seg_per_shard = c.vocab_segments / p.shards;
  const int64_t H = c.hidden_size;
  int64_t launch_no = 0;
  for (size_t b = 0; b < p.batches.size(); ++b) {
    for (const RowRange& ch : p.chunks[b]) {
      for (int sh = 0; sh < p.shards; ++sh) {
        const int s0 = sh * seg_per_shard, s1 = s0 + seg_per_shard;
        const int64_t w_row0 = (int64_t)s0 * g.seg_len;
        const void* Wsh = static_cast<const uint16_t*>(W_lm) + w_row0 * H;
        const bool timed = events && 2 * launch_no + 1 < (int64_t)num_events;
        if (timed) {
          e = hipEventRecord(static_cast<hipEvent_t>(events[2 * launch_no]), s);
          if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
        }
        st = run_rows(h, g, hidden, Wsh, w_row0, targets, rms_gamma, m, ws, T, 0, ch.begin,
                      ch.end, s0, s1, layout->token_tile, sh == 0, s);
        if (st != RLK_OK) return st;
        if (timed) {
          e = hipEventRecord(static_cast<hipEvent_t>(events[2 * launch_no + 1]), s);
          if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
        }
        ++launch_no;
      }
    }
  }
  // One fold over all rows of the call, after every batch's LM-head launches: the per-row
  // arithmetic does not depend on which launch wrote a row's tile partials, so folding all of the
  // call's batches at once gives each row the bits a fold per batch would (and 1 launch, not one
  // per batch).
  {
    const RowRange br{0, T};
    const int64_t n = T;
    rlk::FoldArgs f;
    f.part_m = reinterpret_cast<const float*>(ws + m.pm) + br.begin;
    f.part_s = reinterpret_cast<const float*>(ws + m.ps) + br.begin;
    f.part_u = ent ? reinterpret_cast<const float*>(ws + m.pu) + br.begin : nullptr;
    f.tgt = reinterpret_cast<const float*>(ws + m.tgt) + br.begin;
    f.targets = targets + br.begin;
    f.rec = reinterpret_cast<rlk_segment_record_t*>(ws + m.rec) + br.begin;
    f.ld = T;
    f.rec_ld = T;
    f.seg_len = g.seg_len;
    f.rows = (int32_t)n;
    f.tiles_per_seg = g.tiles_per_seg;
    f.seg_begin = 0;
    f.n_seg = c.vocab_segments;
    f.g_base = 0;
    f.portable = (c.flags & RLK_FLAG_PORTABLE_EXP) ? 1 : 0;
    // the fold of each row block's last segment also merges the segments (C9, C10)
    f.done = done;
    rlk::MergeArgs& mg = f.mg;
    mg.rec = reinterpret_cast<const rlk_segment_record_t*>(ws + m.rec) + br.begin;
    mg.targets = targets + br.begin;
    mg.logp = logp + br.begin;
    mg.lse = lse + br.begin;
    mg.entropy = ent ? entropy + br.begin : nullptr;
    mg.status = status;
    mg.rec_ld = T;
    mg.seg_len = g.seg_len;
    mg.vocab = c.vocab_size;
    mg.rows = (int32_t)n;
    mg.n_seg = c.vocab_segments;
    mg.portable = f.portable;
    e = rlk::launch_fold(f, ent, s);
    if (e != hipSuccess) return hip_fail(e, "segment fold launch");
  }
  return ok();
}

}  // namespace

RLK_API rlk_status_t rlk_logprob_forward(rlk_logprob_t h, const void* hidden, const void* W_lm,
                                         const int32_t* targets, const rlk_layout_desc_t* layout,
                                         const void* rms_gamma, float* logp, float* lse,
                                         float* entropy, void* workspace, size_t workspace_bytes,
                                         rlk_stream_t stream) {
  return forward_impl(h, hidden, W_lm, targets, layout, rms_gamma, logp, lse, entropy, workspace,
                      workspace_bytes, stream, nullptr, 0);
}

RLK_API rlk_status_t rlk_logprob_forward_timed(rlk_logprob_t h, const void* hidden,
                                               const void* W_lm, const int32_t* targets,
                                               const rlk_layout_desc_t* layout,
                                               const void* rms_gamma, float* logp, float* lse,
                                               float* entropy, void* workspace,
                                               size_t workspace_bytes, rlk_stream_t stream,
                                               void* const* events, int32_t num_events) {
  if (num_events < 0 || (num_events > 0 && !events))
    return fail(RLK_ERR_INVALID_ARGUMENT, "events must hold num_events >= 0 entries");
  return forward_impl(h, hidden, W_lm, targets, layout, rms_gamma, logp, lse, entropy, workspace,
                      workspace_bytes, stream, events, num_events);
}

RLK_API rlk_status_t rlk_logprob_forward_noalloc(rlk_logprob_t h, const void* hidden,
                                                 const void* W_lm, const int32_t* targets,
                                                 const rlk_layout_desc_t* layout,
                                                 const void* rms_gamma, float* logp, float* lse,
                                                 float* entropy, rlk_stream_t stream) {
  if (!h) return fail(RLK_ERR_INVALID_ARGUMENT, "handle is NULL");
  size_t need = 0;
  rlk_status_t st = rlk_logprob_workspace_size(&h->cfg, layout, &need);
  if (st != RLK_OK) return st;
  if (need > kScratchBytes)
    return fail(RLK_ERR_WORKSPACE,
                "this forward needs %zu bytes of workspace; the allocation-free entry point has "
                "%zu (use rlk_logprob_forward with a caller workspace, or fewer rows per call)",
                need, kScratchBytes);
  if (!h->scratch) return fail(RLK_ERR_WORKSPACE, "no device scratch for device %d", h->device);
  return forward_impl(h, hidden, W_lm, targets, layout, rms_gamma, logp, lse, entropy, h->scratch,
                      kScratchBytes, stream, nullptr, 0);
}

RLK_API rlk_status_t rlk_logprob_partials_workspace_size(const rlk_logprob_config_t* config,
                                                         int64_t num_rows, int64_t vocab_begin,
                                                         int64_t vocab_end, size_t* bytes) {
  if (!bytes) return fail(RLK_ERR_INVALID_ARGUMENT, "bytes is NULL");
  rlk_status_t st = check_config(config);
  if (st != RLK_OK) return st;
  if (num_rows < 0 || num_rows > 0x7fffffffLL)
    return fail(RLK_ERR_INVALID_ARGUMENT, "num_rows out of range");
  const Geometry g = geometry(*config);
  if (vocab_begin < 0 || vocab_end > config->vocab_size || vocab_end <= vocab_begin ||
      vocab_begin % g.seg_len != 0 || vocab_end % g.seg_len != 0)
    return fail(RLK_ERR_CONTRACT, "vocab range [%lld, %lld) is not on segment boundaries of %lld",
                (long long)vocab_begin, (long long)vocab_end, (long long)g.seg_len);
  const int nseg = (int)((vocab_end - vocab_begin) / g.seg_len);
  *bytes = ws_map(*config, num_rows, nseg * g.tiles_per_seg, 0).total;
  return ok();
}

RLK_API rlk_status_t rlk_logprob_partials(rlk_logprob_t h, const void* hidden,
                                          const void* W_shard, int64_t vocab_begin,
                                          int64_t vocab_end, const int32_t* targets,
                                          int64_t num_rows, const void* rms_gamma,
                                          rlk_segment_record_t* records, void* workspace,
                                          size_t workspace_bytes, rlk_stream_t stream) {
  if (!h) return fail(RLK_ERR_INVALID_ARGUMENT, "handle is NULL");
  const rlk_logprob_config_t& c = h->cfg;
  size_t need = 0;
  rlk_status_t st = rlk_logprob_partials_workspace_size(&c, num_rows, vocab_begin, vocab_end, &need);
  if (st != RLK_OK) return st;
  const bool ent = c.flags & RLK_FLAG_ENTROPY;
  const bool rms = c.flags & RLK_FLAG_RMSNORM;
  if (num_rows > 0) {
    if (!hidden || !W_shard || !targets || !records)
      return fail(RLK_ERR_INVALID_ARGUMENT, "hidden, W_shard, targets and records are required");
    if (rms && !rms_gamma) return fail(RLK_ERR_INVALID_ARGUMENT, "rms_gamma required");
    if (!aligned16(hidden) || !aligned16(W_shard) || !aligned16(targets) || !aligned16(records) ||
        (rms_gamma && !aligned16(rms_gamma)))
      return fail(RLK_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
  }
  if (!rms && rms_gamma) return fail(RLK_ERR_CONTRACT, "rms_gamma given but RLK_FLAG_RMSNORM not set");
  if (!workspace || workspace_bytes < need)
    return fail(RLK_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(RLK_ERR_ALIGNMENT, "workspace must be 256-byte aligned");
  if (num_rows == 0) return ok();
  DeviceGuard guard(h->device);
  if (guard.err != hipSuccess) return hip_fail(guard.err, "hipSetDevice");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Geometry g = geometry(c);
  const int s0 = (int)(vocab_begin / g.seg_len), s1 = (int)(vocab_end / g.seg_len);
  const WsMap m = ws_map(c, num_rows, (s1 - s0) * g.tiles_per_seg, 0);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const int g_base = s0 * g.tiles_per_seg;
  hipError_t e = rlk::launch_clear_status(reinterpret_cast<uint32_t*>(ws + m.status), nullptr, 0, s);
  if (e != hipSuccess) return hip_fail(e, "status clear launch");
  st = run_rows(h, g, hidden, W_shard, vocab_begin, targets, rms_gamma, m, ws, num_rows, g_base, 0,
                num_rows, s0, s1, 0, true, s);
  if (st != RLK_OK) return st;
  rlk::FoldArgs f;
  f.part_m = reinterpret_cast<const float*>(ws + m.pm);
  f.part_s = reinterpret_cast<const float*>(ws + m.ps);
  f.part_u = ent ? reinterpret_cast<const float*>(ws + m.pu) : nullptr;
  f.tgt = reinterpret_cast<const float*>(ws + m.tgt);
  f.targets = targets;
  f.rec = records;
  f.ld = num_rows;
  f.rec_ld = num_rows;
  f.seg_len = g.seg_len;
  f.rows = (int32_t)num_rows;
  f.tiles_per_seg = g.tiles_per_seg;
  f.seg_begin = s0;
  f.n_seg = s1 - s0;
  f.g_base = g_base;
  f.portable = (c.flags & RLK_FLAG_PORTABLE_EXP) ? 1 : 0;
  f.done = nullptr;  // records only: the merge runs after the shards are gathered
  f.mg = rlk::MergeArgs{};
  e = rlk::launch_fold(f, ent, s);
  if (e != hipSuccess) return hip_fail(e, "segment fold launch");
  return ok();
}

RLK_API rlk_status_t rlk_logprob_merge(rlk_logprob_t h, const rlk_segment_record_t* records,
                                       const int32_t* targets, int64_t num_rows, float* logp,
                                       float* lse, float* entropy, uint32_t* status,
                                       rlk_stream_t stream) {
  if (!h) return fail(RLK_ERR_INVALID_ARGUMENT, "handle is NULL");
  const rlk_logprob_config_t& c = h->cfg;
  const bool ent = c.flags & RLK_FLAG_ENTROPY;
  if (num_rows < 0 || num_rows > 0x7fffffffLL)
    return fail(RLK_ERR_INVALID_ARGUMENT, "num_rows out of range");
  if (num_rows == 0) return ok();
  if (!records || !targets || !logp || !lse)
    return fail(RLK_ERR_INVALID_ARGUMENT, "records, targets, logp and lse are required");
  if (ent && !entropy) return fail(RLK_ERR_INVALID_ARGUMENT, "entropy output required");
  if (!ent && entropy) return fail(RLK_ERR_CONTRACT, "entropy given but RLK_FLAG_ENTROPY not set");
  if (!aligned16(records) || !aligned16(targets) || !aligned16(logp) || !aligned16(lse) ||
      (entropy && !aligned16(entropy)) || (reinterpret_cast<uintptr_t>(status) & 3u))
    return fail(RLK_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
  DeviceGuard guard(h->device);
  if (guard.err != hipSuccess) return hip_fail(guard.err, "hipSetDevice");
  const Geometry g = geometry(c);
  rlk::MergeArgs mg;
  mg.rec = records;
  mg.targets = targets;
  mg.logp = logp;
  mg.lse = lse;
  mg.entropy = entropy;
  mg.status = status;
  mg.rec_ld = num_rows;
  mg.seg_len = g.seg_len;
  mg.vocab = c.vocab_size;
  mg.rows = (int32_t)num_rows;
  mg.n_seg = c.vocab_segments;
  mg.portable = (c.flags & RLK_FLAG_PORTABLE_EXP) ? 1 : 0;
  hipError_t e = rlk::launch_merge(mg, ent, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  return ok();
}

RLK_API rlk_status_t rlk_logprob_device_status(rlk_logprob_t h, const void* workspace,
                                               rlk_stream_t stream, uint32_t* flags) {
  if (!h || !workspace || !flags) return fail(RLK_ERR_INVALID_ARGUMENT, "NULL argument");
  DeviceGuard guard(h->device);
  if (guard.err != hipSuccess) return hip_fail(guard.err, "hipSetDevice");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  uint32_t v = 0;
  e = hipMemcpy(&v, workspace, 4, hipMemcpyDeviceToHost);  // status word sits at offset 0
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy status");
  *flags = v;
  return ok();
}

// ============================================================================================
// Backward (B1-B3 in rlk_backward.hip)
// ============================================================================================
namespace {

struct BwdMap {
  int64_t L, Lp, J;    // segment length, padded length, padded vocab width S_c Lp
  int64_t chunk;       // rows per chunk
  size_t status, dz, dpart, y, dy, r, gp, total;
};

// Rows per chunk: the caller's row_chunk (or all rows), capped so that the dz rows of a chunk
// span less than 2 GiB (the 32-bit range of the GEMMs' buffer descriptors). Any multiple of 128
// gives the same bits (B3, B4), so the cap changes no result.
int64_t bwd_chunk(int64_t rows, int64_t row_chunk, int64_t J) {
  const int64_t r = std::max<int64_t>(rows, 1);
  int64_t c = row_chunk > 0 ? std::min<int64_t>(row_chunk, r) : r;
  const int64_t cap = std::max<int64_t>((0x7fffffffLL / (2 * J)) / rlk::kBwdKPad * rlk::kBwdKPad,
                                        rlk::kBwdKPad);
  return std::min(c, cap);
}

// want_h: a gradient w.r.t. the LM-head input is needed (grad_hidden, or grad_gamma through the
// RMSNorm); nseg: the vocab segments processed (all of them, or a shard's); shard: the dh
// partials go to the caller (no tree, no RMSNorm backward here).
BwdMap bwd_map(const rlk_logprob_config_t& c, int64_t rows, int64_t row_chunk, bool want_h,
               int nseg = 0, bool shard = false) {
  BwdMap m;
  const int S = nseg > 0 ? nseg : c.vocab_segments;
  m.L = c.vocab_size / c.vocab_segments;
  m.Lp = (int64_t)round_up((size_t)m.L, rlk::kBwdKPad);
  m.J = S * m.Lp;
  m.chunk = bwd_chunk(rows, row_chunk, m.J);
  const size_t H = (size_t)c.hidden_size;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = round_up(off + bytes, 256);
    return at;
  };
  m.status = take(rlk::kStatusSlotWords * 4);  // the GEMMs' work queues (from word kQueueWord)
  m.dz = take((size_t)m.chunk * (size_t)m.J * 2);
  m.dpart = (want_h && S > 1 && !shard) ? take((size_t)S * (size_t)m.chunk * H * 4) : 0;
  const bool rms = c.flags & RLK_FLAG_RMSNORM;
  const bool rms_bwd = rms && want_h && !shard;
  m.y = rms ? take((size_t)m.chunk * H * 2) : 0;
  m.dy = rms_bwd ? take((size_t)m.chunk * H * 4) : 0;
  m.r = rms_bwd ? take((size_t)m.chunk * 4) : 0;
  m.gp = rms_bwd ? take((size_t)((m.chunk + rlk::kGammaGroup - 1) / rlk::kGammaGroup) * H * 4) : 0;
  m.total = std::max<size_t>(off, 256);
  return m;
}

rlk_status_t check_bwd_rows(const rlk_logprob_config_t& c, int64_t num_rows, int64_t row_chunk) {
  if (num_rows < 0 || num_rows > 0x7fffffffLL)
    return fail(RLK_ERR_INVALID_ARGUMENT, "num_rows out of range");
  if (row_chunk < 0 || (row_chunk > 0 && row_chunk % rlk::kBwdKPad != 0))
    return fail(RLK_ERR_UNSUPPORTED_SHAPE, "row_chunk %lld is not 0 or a positive multiple of %d",
                (long long)row_chunk, rlk::kBwdKPad);
  const BwdMap m = bwd_map(c, num_rows, row_chunk, true);
  // 32-bit buffer ranges: one vocab segment of W (the dh GEMM's K-major operand), 256 rows of
  // dz, and 128 rows of dz
  if (m.Lp * (int64_t)c.hidden_size * 2 >= 0x7fffffffLL || 256 * m.J * 2 >= 0x7fffffffLL ||
      (int64_t)rlk::kBwdKPad * m.J * 2 >= 0x7fffffffLL)
    return fail(RLK_ERR_UNSUPPORTED_SHAPE, "vocab segment x hidden size too large for the backward");
  return RLK_OK;
}

// Arguments of one backward run over the vocab segments [s0, s1) (all of them, or a shard's).
struct BwdRun {
  const uint16_t* hidden;
  const uint16_t* W;  // W_lm rows from s0 L on
  int s0, s1;
  const int32_t* targets;
  int64_t T;
  const uint16_t* gamma;
  const float *lse, *entropy, *g, *gH;
  float* grad_hidden;  // full run only
  float* grad_W;       // rows of the range
  float* grad_gamma;   // full run only
  float* parts;        // shard run: per-segment dh partials [s1 - s0][T][H]
  bool accumulate;
  int64_t row_chunk;
};

rlk_status_t backward_run(const rlk_logprob* h, const BwdRun& b, void* workspace,
                            size_t workspace_bytes, hipStream_t s) {
  const rlk_logprob_config_t& c = h->cfg;
  const int64_t num_rows = b.T;
  const bool rms = c.flags & RLK_FLAG_RMSNORM;
  const bool shard = b.parts != nullptr;
  const bool want_x = b.grad_hidden != nullptr, want_w = b.grad_W != nullptr;
  const bool want_g = b.grad_gamma != nullptr;
  const bool want_h = want_x || want_g || shard;
  const int nseg = b.s1 - b.s0;
  const BwdMap m = bwd_map(c, num_rows, b.row_chunk, want_h, nseg, shard);
  if (!workspace || workspace_bytes < m.total)
    return fail(RLK_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", m.total,
                workspace_bytes);
  DeviceGuard guard(h->device);
  if (guard.err != hipSuccess) return hip_fail(guard.err, "hipSetDevice");
  const bool accumulate = b.accumulate;
  const int S = nseg;
  const int H = c.hidden_size;
  const int64_t Vr = (int64_t)nseg * m.L;  // vocab rows of the range (of W_lm or the shard)
  float* const grad_W = b.grad_W;
  float* const grad_gamma = b.grad_gamma;
  float* const grad_hidden = b.grad_hidden;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  hipError_t e;
  if (num_rows == 0) {
    if (want_w && !accumulate) {
      e = rlk::launch_zero_f32(grad_W, Vr * H, s);
      if (e != hipSuccess) return hip_fail(e, "zero launch");
    }
    if (want_g && !accumulate) {
      e = rlk::launch_zero_f32(grad_gamma, H, s);
      if (e != hipSuccess) return hip_fail(e, "zero launch");
    }
    return ok();
  }
  uint16_t* dz = reinterpret_cast<uint16_t*>(ws + m.dz);
  float* dpart = reinterpret_cast<float*>(ws + m.dpart);
  uint16_t* ynorm = reinterpret_cast<uint16_t*>(ws + m.y);
  float* dy = reinterpret_cast<float*>(ws + m.dy);
  float* rrow = reinterpret_cast<float*>(ws + m.r);
  float* gpart = reinterpret_cast<float*>(ws + m.gp);
  const uint16_t* gam = b.gamma;
  const uint16_t* hid = b.hidden;
  const uint16_t* Wb = b.W;
  // the persistent GEMMs' work queues: zero before the first, and each launch leaves them zero
  uint32_t* queue = reinterpret_cast<uint32_t*>(ws + m.status) + rlk::kQueueWord;
  e = rlk::launch_clear_status(reinterpret_cast<uint32_t*>(ws + m.status), nullptr, 0, s);
  if (e != hipSuccess) return hip_fail(e, "clear launch");
  int64_t chunk_no = 0;
  for (int64_t r0 = 0; r0 < num_rows; r0 += m.chunk, ++chunk_no) {
    const int64_t r1 = std::min<int64_t>(num_rows, r0 + m.chunk);
    const int64_t n = r1 - r0;
    const int64_t np = (int64_t)round_up((size_t)n, rlk::kBwdKPad);
    // the LM-head input of these rows: the hidden rows, or their RMSNorm (C12, recomputed)
    const uint16_t* hin = hid + r0 * H;
    if (rms) {
      rlk::RmsArgs ra;
      ra.x = hin;
      ra.gamma = gam;
      ra.y = ynorm;
      ra.rows = (int32_t)n;
      ra.H = H;
      ra.inv_H = 1.0f / (float)H;
      ra.eps = c.rms_eps;
      ra.portable = (c.flags & RLK_FLAG_PORTABLE_EXP) ? 1 : 0;
      e = rlk::launch_rmsnorm(ra, s);
      if (e != hipSuccess) return hip_fail(e, "rmsnorm launch");
      hin = ynorm;
    }
    // B1: dz over the segment-padded positions (it writes the padding zeros)
    rlk::GemmArgs a{};
    a.A = Wb;
    a.lda = H;
    a.B = hin;
    a.ldb = H;
    a.M = (int32_t)m.J;
    a.N = (int32_t)n;
    a.K = H;
    a.seg_len = m.L;
    a.seg_pad = m.Lp;
    a.targets = b.targets + r0;
    a.lse = b.lse + r0;
    a.ent = b.gH ? b.entropy + r0 : nullptr;
    a.g = b.g + r0;
    a.gH = b.gH ? b.gH + r0 : nullptr;
    a.dz = dz;
    a.lddz = m.J;
    a.v_base = (int64_t)b.s0 * m.L;
    a.inv_tau = c.inv_temperature;
    a.portable = (c.flags & RLK_FLAG_PORTABLE_EXP) ? 1 : 0;
    a.queue = queue;
    a.n_cu = h->n_cu;
    e = rlk::launch_gemm_dz(a, s);
    if (e != hipSuccess) return hip_fail(e, "dz launch");
    if (want_h) {
      // B2: per segment one chain over its positions (W read K-major, rows past the segment read
      // as zeros), then the segment tree
      rlk::GemmArgs g{};
      g.A = Wb;
      g.lda = H;
      g.a_batch = m.L * H;
      g.ka_rows = m.L;
      g.B = dz;
      g.ldb = m.J;
      g.b_batch = m.Lp;
      g.M = H;
      g.N = (int32_t)n;
      g.K = (int32_t)m.Lp;
      float* dh = rms ? dy : grad_hidden + r0 * H;
      if (shard) {
        // a shard's per-segment partials, before the tree: parts[s - s0][t][k]
        g.C = b.parts + r0 * H;
        g.c_batch = num_rows * H;
      } else {
        g.C = S > 1 ? dpart : dh;
        g.c_batch = n * H;
      }
      g.ldc = H;
      g.queue = queue;
      g.n_cu = h->n_cu;
      e = rlk::launch_gemm_out(g, S, false, s);
      if (e != hipSuccess) return hip_fail(e, "dh launch");
      if (S > 1 && !shard) {
        e = rlk::launch_seg_tree(dpart, n * H, S, dh, n * H, s);
        if (e != hipSuccess) return hip_fail(e, "dh tree launch");
      }
      if (rms && !shard) {
        // B4: through the RMSNorm to its input, and the gamma gradient
        rlk::RmsBwdArgs rb;
        rb.x = hid + r0 * H;
        rb.gamma = gam;
        rb.dy = dy;
        rb.dx = want_x ? grad_hidden + r0 * H : nullptr;
        rb.r = rrow;
        rb.rows = (int32_t)n;
        rb.H = H;
        rb.inv_H = 1.0f / (float)H;
        rb.eps = c.rms_eps;
        rb.portable = (c.flags & RLK_FLAG_PORTABLE_EXP) ? 1 : 0;
        e = rlk::launch_rmsnorm_bwd(rb, s);
        if (e != hipSuccess) return hip_fail(e, "rmsnorm backward launch");
        if (want_g) {
          e = rlk::launch_dgamma(dy, hid + r0 * H, rrow, gpart, (int)n, H, grad_gamma,
                                 accumulate || chunk_no > 0, s);
          if (e != hipSuccess) return hip_fail(e, "dgamma launch");
        }
      }
    }
    if (want_w) {
      // B3: the hidden rows and dz read K-major (K = row, rows past the chunk read as zeros);
      // the chain over rows continues from the previous chunk
      rlk::GemmArgs g{};
      g.A = hin;
      g.lda = H;
      g.ka_rows = n;
      g.B = dz;
      g.ldb = m.J;
      g.kb_rows = n;
      g.M = H;
      g.N = (int32_t)m.J;
      g.K = (int32_t)np;
      g.seg_len = m.L;
      g.seg_pad = m.Lp;
      g.C = grad_W;
      g.ldc = H;
      g.accumulate = (accumulate || chunk_no > 0) ? 1 : 0;
      g.map_rows = 1;
      g.queue = queue;
      g.n_cu = h->n_cu;
      e = rlk::launch_gemm_out(g, 1, true, s);
      if (e != hipSuccess) return hip_fail(e, "dW launch");
    }
  }
  return ok();
}

}  // namespace

RLK_API rlk_status_t rlk_logprob_backward_workspace_size(const rlk_logprob_config_t* config,
                                                         int64_t num_rows, int64_t row_chunk,
                                                         size_t* bytes) {
  if (!bytes) return fail(RLK_ERR_INVALID_ARGUMENT, "bytes is NULL");
  rlk_status_t st = check_config(config);
  if (st != RLK_OK) return st;
  st = check_bwd_rows(*config, num_rows, row_chunk);
  if (st != RLK_OK) return st;
  *bytes = bwd_map(*config, num_rows, row_chunk, true).total;
  return ok();
}

RLK_API rlk_status_t rlk_logprob_backward(rlk_logprob_t h, const void* hidden, const void* W_lm,
                                          const int32_t* targets, int64_t num_rows,
                                          const void* rms_gamma, const float* lse,
                                          const float* entropy, const float* grad_logp,
                                          const float* grad_entropy, float* grad_hidden,
                                          float* grad_W, float* grad_gamma, uint32_t flags,
                                          int64_t row_chunk, void* workspace,
                                          size_t workspace_bytes, rlk_stream_t stream) {
  if (!h) return fail(RLK_ERR_INVALID_ARGUMENT, "handle is NULL");
  const rlk_logprob_config_t& c = h->cfg;
  if (flags & ~RLK_BWD_ACCUMULATE)
    return fail(RLK_ERR_INVALID_ARGUMENT, "unknown flag bits 0x%x", flags);
  rlk_status_t st = check_bwd_rows(c, num_rows, row_chunk);
  if (st != RLK_OK) return st;
  const bool rms = c.flags & RLK_FLAG_RMSNORM;
  if (!rms && (rms_gamma || grad_gamma))
    return fail(RLK_ERR_CONTRACT, "rms_gamma / grad_gamma given but RLK_FLAG_RMSNORM not set");
  if (rms && num_rows > 0 && !rms_gamma)
    return fail(RLK_ERR_INVALID_ARGUMENT, "rms_gamma is required with RLK_FLAG_RMSNORM");
  const bool want_x = grad_hidden != nullptr, want_w = grad_W != nullptr;
  const bool want_g = grad_gamma != nullptr;
  const bool want_h = want_x || want_g;  // a gradient w.r.t. the LM-head input is needed
  if (!want_x && !want_w && !want_g) return fail(RLK_ERR_INVALID_ARGUMENT, "no gradient requested");
  if (grad_entropy && !(c.flags & RLK_FLAG_ENTROPY))
    return fail(RLK_ERR_CONTRACT, "grad_entropy given but RLK_FLAG_ENTROPY not set");
  if (grad_entropy && !entropy)
    return fail(RLK_ERR_INVALID_ARGUMENT, "grad_entropy needs the forward's entropy");
  if (num_rows > 0 && (!hidden || !W_lm || !targets || !lse || !grad_logp))
    return fail(RLK_ERR_INVALID_ARGUMENT, "hidden, W, targets, lse and grad_logp are required");
  if (!W_lm && want_w) return fail(RLK_ERR_INVALID_ARGUMENT, "W is required");
  if (!aligned16(hidden) || !aligned16(W_lm) || !aligned16(targets) || !aligned16(lse) ||
      !aligned16(grad_logp) || !aligned16(entropy) || !aligned16(grad_entropy) ||
      !aligned16(grad_hidden) || !aligned16(grad_W) || !aligned16(workspace) ||
      !aligned16(rms_gamma) || !aligned16(grad_gamma))
    return fail(RLK_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
  BwdRun b;
  b.hidden = static_cast<const uint16_t*>(hidden);
  b.W = static_cast<const uint16_t*>(W_lm);
  b.s0 = 0;
  b.s1 = c.vocab_segments;
  b.targets = targets;
  b.T = num_rows;
  b.gamma = static_cast<const uint16_t*>(rms_gamma);
  b.lse = lse;
  b.entropy = entropy;
  b.g = grad_logp;
  b.gH = grad_entropy;
  b.grad_hidden = grad_hidden;
  b.grad_W = grad_W;
  b.grad_gamma = grad_gamma;
  b.parts = nullptr;
  b.accumulate = flags & RLK_BWD_ACCUMULATE;
  b.row_chunk = row_chunk;
  return backward_run(h, b, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

// ---- the backward of one vocab shard, and the merge of the shards' dh partials ----
namespace {

rlk_status_t check_shard_range(const rlk_logprob_config_t& c, int64_t vocab_begin,
                               int64_t vocab_end, int* s0, int* s1) {
  const Geometry g = geometry(c);
  if (vocab_begin < 0 || vocab_end > c.vocab_size || vocab_end <= vocab_begin ||
      vocab_begin % g.seg_len != 0 || vocab_end % g.seg_len != 0)
    return fail(RLK_ERR_CONTRACT, "vocab range [%lld, %lld) is not on segment boundaries of %lld",
                (long long)vocab_begin, (long long)vocab_end, (long long)g.seg_len);
  *s0 = (int)(vocab_begin / g.seg_len);
  *s1 = (int)(vocab_end / g.seg_len);
  return RLK_OK;
}

// merge workspace: dy [T][H] fp32, r [T], dgamma group sums (RMSNorm only)
struct MergeMap {
  size_t dy, r, gp, total;
};
MergeMap merge_map(const rlk_logprob_config_t& c, int64_t rows) {
  MergeMap m{};
  const size_t H = (size_t)c.hidden_size;
  const size_t T = (size_t)std::max<int64_t>(rows, 1);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = round_up(off + bytes, 256);
    return at;
  };
  if (c.flags & RLK_FLAG_RMSNORM) {
    m.dy = take(T * H * 4);
    m.r = take(T * 4);
    m.gp = take((T + rlk::kGammaGroup - 1) / rlk::kGammaGroup * H * 4);
  }
  m.total = std::max<size_t>(off, 256);
  return m;
}

}  // namespace

RLK_API rlk_status_t rlk_logprob_backward_partials_workspace_size(
    const rlk_logprob_config_t* config, int64_t num_rows, int64_t vocab_begin, int64_t vocab_end,
    int64_t row_chunk, size_t* bytes) {
  if (!bytes) return fail(RLK_ERR_INVALID_ARGUMENT, "bytes is NULL");
  rlk_status_t st = check_config(config);
  if (st != RLK_OK) return st;
  st = check_bwd_rows(*config, num_rows, row_chunk);
  if (st != RLK_OK) return st;
  int s0, s1;
  st = check_shard_range(*config, vocab_begin, vocab_end, &s0, &s1);
  if (st != RLK_OK) return st;
  *bytes = bwd_map(*config, num_rows, row_chunk, true, s1 - s0, true).total;
  return ok();
}

RLK_API rlk_status_t rlk_logprob_backward_partials(
    rlk_logprob_t h, const void* hidden, const void* W_shard, int64_t vocab_begin,
    int64_t vocab_end, const int32_t* targets, int64_t num_rows, const void* rms_gamma,
    const float* lse, const float* entropy, const float* grad_logp, const float* grad_entropy,
    float* dh_parts, float* grad_W_shard, uint32_t flags, int64_t row_chunk, void* workspace,
    size_t workspace_bytes, rlk_stream_t stream) {
  if (!h) return fail(RLK_ERR_INVALID_ARGUMENT, "handle is NULL");
  const rlk_logprob_config_t& c = h->cfg;
  if (flags & ~RLK_BWD_ACCUMULATE)
    return fail(RLK_ERR_INVALID_ARGUMENT, "unknown flag bits 0x%x", flags);
  rlk_status_t st = check_bwd_rows(c, num_rows, row_chunk);
  if (st != RLK_OK) return st;
  int s0, s1;
  st = check_shard_range(c, vocab_begin, vocab_end, &s0, &s1);
  if (st != RLK_OK) return st;
  const bool rms = c.flags & RLK_FLAG_RMSNORM;
  if (!rms && rms_gamma)
    return fail(RLK_ERR_CONTRACT, "rms_gamma given but RLK_FLAG_RMSNORM not set");
  if (rms && num_rows > 0 && !rms_gamma)
    return fail(RLK_ERR_INVALID_ARGUMENT, "rms_gamma is required with RLK_FLAG_RMSNORM");
  if (!dh_parts) return fail(RLK_ERR_INVALID_ARGUMENT, "dh_parts is required");
  if (grad_entropy && !(c.flags & RLK_FLAG_ENTROPY))
    return fail(RLK_ERR_CONTRACT, "grad_entropy given but RLK_FLAG_ENTROPY not set");
  if (grad_entropy && !entropy)
    return fail(RLK_ERR_INVALID_ARGUMENT, "grad_entropy needs the forward's entropy");
  if (num_rows > 0 && (!hidden || !W_shard || !targets || !lse || !grad_logp))
    return fail(RLK_ERR_INVALID_ARGUMENT, "hidden, W_shard, targets, lse and grad_logp are required");
  if (!aligned16(hidden) || !aligned16(W_shard) || !aligned16(targets) || !aligned16(lse) ||
      !aligned16(grad_logp) || !aligned16(entropy) || !aligned16(grad_entropy) ||
      !aligned16(dh_parts) || !aligned16(grad_W_shard) || !aligned16(workspace) ||
      !aligned16(rms_gamma))
    return fail(RLK_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
  if (num_rows == 0) return ok();
  BwdRun b;
  b.hidden = static_cast<const uint16_t*>(hidden);
  b.W = static_cast<const uint16_t*>(W_shard);
  b.s0 = s0;
  b.s1 = s1;
  b.targets = targets;
  b.T = num_rows;
  b.gamma = static_cast<const uint16_t*>(rms_gamma);
  b.lse = lse;
  b.entropy = entropy;
  b.g = grad_logp;
  b.gH = grad_entropy;
  b.grad_hidden = nullptr;
  b.grad_W = grad_W_shard;
  b.grad_gamma = nullptr;
  b.parts = dh_parts;
  b.accumulate = flags & RLK_BWD_ACCUMULATE;
  b.row_chunk = row_chunk;
  return backward_run(h, b, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

RLK_API rlk_status_t rlk_logprob_backward_merge_workspace_size(const rlk_logprob_config_t* config,
                                                               int64_t num_rows, size_t* bytes) {
  if (!bytes) return fail(RLK_ERR_INVALID_ARGUMENT, "bytes is NULL");
  rlk_status_t st = check_config(config);
  if (st != RLK_OK) return st;
  if (num_rows < 0 || num_rows > 0x7fffffffLL)
    return fail(RLK_ERR_INVALID_ARGUMENT, "num_rows out of range");
  *bytes = merge_map(*config, num_rows).total;
  return ok();
}

RLK_API rlk_status_t rlk_logprob_backward_merge(rlk_logprob_t h, const float* dh_parts,
                                                const void* hidden, const void* rms_gamma,
                                                int64_t num_rows, float* grad_hidden,
                                                float* grad_gamma, uint32_t flags,
                                                void* workspace, size_t workspace_bytes,
                                                rlk_stream_t stream) {
  if (!h) return fail(RLK_ERR_INVALID_ARGUMENT, "handle is NULL");
  const rlk_logprob_config_t& c = h->cfg;
  if (flags & ~RLK_BWD_ACCUMULATE)
    return fail(RLK_ERR_INVALID_ARGUMENT, "unknown flag bits 0x%x", flags);
  if (num_rows < 0 || num_rows > 0x7fffffffLL)
    return fail(RLK_ERR_INVALID_ARGUMENT, "num_rows out of range");
  const bool rms = c.flags & RLK_FLAG_RMSNORM;
  if (!rms && (rms_gamma || grad_gamma))
    return fail(RLK_ERR_CONTRACT, "rms_gamma / grad_gamma given but RLK_FLAG_RMSNORM not set");
  if (rms && num_rows > 0 && (!rms_gamma || !hidden))
    return fail(RLK_ERR_INVALID_ARGUMENT, "hidden and rms_gamma are required with RLK_FLAG_RMSNORM");
  if (!grad_hidden && !grad_gamma) return fail(RLK_ERR_INVALID_ARGUMENT, "no gradient requested");
  if (num_rows > 0 && !dh_parts) return fail(RLK_ERR_INVALID_ARGUMENT, "dh_parts is required");
  if (!rms && !grad_hidden) return fail(RLK_ERR_INVALID_ARGUMENT, "grad_hidden is required");
  if (!aligned16(dh_parts) || !aligned16(hidden) || !aligned16(rms_gamma) ||
      !aligned16(grad_hidden) || !aligned16(grad_gamma) || !aligned16(workspace))
    return fail(RLK_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
  const MergeMap m = merge_map(c, num_rows);
  if (!workspace || workspace_bytes < m.total)
    return fail(RLK_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", m.total,
                workspace_bytes);
  DeviceGuard guard(h->device);
  if (guard.err != hipSuccess) return hip_fail(guard.err, "hipSetDevice");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int H = c.hidden_size;
  const bool accumulate = flags & RLK_BWD_ACCUMULATE;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  hipError_t e;
  if (num_rows == 0) {
    if (grad_gamma && !accumulate) {
      e = rlk::launch_zero_f32(grad_gamma, H, s);
      if (e != hipSuccess) return hip_fail(e, "zero launch");
    }
    return ok();
  }
  const int64_t n = num_rows * H;
  // B2's segment tree (B4 then takes it through the RMSNorm)
  float* dh = rms ? reinterpret_cast<float*>(ws + m.dy) : grad_hidden;
  e = rlk::launch_seg_tree(dh_parts, n, c.vocab_segments, dh, n, s);
  if (e != hipSuccess) return hip_fail(e, "dh tree launch");
  if (rms) {
    float* rrow = reinterpret_cast<float*>(ws + m.r);
    rlk::RmsBwdArgs rb;
    rb.x = static_cast<const uint16_t*>(hidden);
    rb.gamma = static_cast<const uint16_t*>(rms_gamma);
    rb.dy = dh;
    rb.dx = grad_hidden;
    rb.r = rrow;
    rb.rows = (int32_t)num_rows;
    rb.H = H;
    rb.inv_H = 1.0f / (float)H;
    rb.eps = c.rms_eps;
    rb.portable = (c.flags & RLK_FLAG_PORTABLE_EXP) ? 1 : 0;
    e = rlk::launch_rmsnorm_bwd(rb, s);
    if (e != hipSuccess) return hip_fail(e, "rmsnorm backward launch");
    if (grad_gamma) {
      e = rlk::launch_dgamma(dh, static_cast<const uint16_t*>(hidden), rrow,
                             reinterpret_cast<float*>(ws + m.gp), (int)num_rows, H, grad_gamma,
                             accumulate, s);
      if (e != hipSuccess) return hip_fail(e, "dgamma launch");
    }
  }
  return ok();
}
