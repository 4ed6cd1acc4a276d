// Work queues of the persistent kernels (the LM-head kernel k_lmhead and the backward GEMMs).
// Host and device code: the launcher sets a launch's item geometry with queue_setup, every block
// maps the claims it makes to items with queue_item, and a host program enumerates every queue to
// check that the items of a launch are handed out exactly once. Q is the launch's argument struct
// (LmheadArgs or GemmArgs), which carries the geometry in its q_* fields.
//
// A launch's items are its (vocab block, row tile) pairs. Row tiles go in bands (the hidden rows
// of a band stay in the MALL while the vocabulary streams past them), one band after the other.
// Inside a band the items are ordered in groups of kGroupVB vocab blocks across all of the band's
// row tiles, vocab block fastest, so that the ~32 items an XCD runs at once share W and hidden
// tiles in its L2; XCD x owns the contiguous items [x per, (x+1) per) of that order,
// per = ceil(items / 8). Queue x lists XCD x's items band after band. Which block computes an
// item never changes its arithmetic, so the schedule never changes a result bit.
#pragma once

#include <stdint.h>

#include "rlk_internal.h"

namespace rlk {

constexpr int kQueues = 8;   // one per XCD
constexpr int kGroupVB = 8;  // vocab blocks per group (measured best of 2, 4, 6, 8, 16)

__host__ __device__ inline int qmin(int a, int b) { return a < b ? a : b; }
__host__ __device__ inline int qmax(int a, int b) { return a > b ? a : b; }

// Item geometry of a launch of n_vb vocab blocks x n_tt row tiles in bands of rb row tiles.
template <class Q>
__host__ __device__ inline void queue_setup(Q& q, int64_t n_vb, int64_t n_tt, int64_t rb) {
  q.q_nvb = (int32_t)n_vb;
  q.q_rb = (int32_t)(rb < n_tt ? rb : n_tt);
  q.q_nfull = (int32_t)(n_tt / q.q_rb);
  q.q_perf = (int32_t)((n_vb * q.q_rb + kQueues - 1) / kQueues);
  q.q_tail_tt = (int32_t)(n_tt - (int64_t)q.q_nfull * q.q_rb);
  q.q_pert = (int32_t)((n_vb * q.q_tail_tt + kQueues - 1) / kQueues);
}

// The c-th item of queue x in (vb, tt); false past the queue's end.
template <class Q>
__host__ __device__ inline bool queue_item(const Q& a, int x, uint32_t c, int& vb, int& tt) {
  const int nvb = a.q_nvb;
  const int len_f = qmax(0, qmin(a.q_perf, nvb * a.q_rb - x * a.q_perf));  // per full band
  const uint32_t c_full = (uint32_t)(a.q_nfull * len_f);
  int band, w, per, nb_tt;
  if (c < c_full) {
    band = (int)(c / (uint32_t)len_f);
    w = (int)c - band * len_f;
    per = a.q_perf;
    nb_tt = a.q_rb;
  } else {
    band = a.q_nfull;
    nb_tt = a.q_tail_tt;
    per = a.q_pert;
    const int len = qmax(0, qmin(per, nvb * nb_tt - x * per));
    if (c - c_full >= (uint32_t)len) return false;
    w = (int)(c - c_full);
  }
  const int L = x * per + w;
  const int grp = L / (kGroupVB * nb_tt);
  const int first_v = grp * kGroupVB;
  const int gsz = qmin(kGroupVB, nvb - first_v);
  const int within = L - grp * kGroupVB * nb_tt;
  vb = first_v + within % gsz;
  tt = band * a.q_rb + within / gsz;
  return true;
}

}  // namespace rlk
