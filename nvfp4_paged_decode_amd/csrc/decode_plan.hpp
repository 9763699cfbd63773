// Balanced split-K over the pages of a whole batch (device side).
//
// The pages of all sequences, concatenated in batch order, form one list of
// P pages (sequence b contributes ceil(L_b / T) of them).  Workgroup w of
// nwg owns pages [floor(w P / nwg), floor((w+1) P / nwg)).  Every range is
// contiguous and ranges are monotone in w, so the (workgroup, sequence)
// pairs that overlap are indexed without collision by w + b: this is the
// partial slot the workgroup writes for that sequence.  Kernels and the
// merge compute the same ranges from seq_lens with the same integer
// arithmetic.
#pragma once

#include "common.hpp"

namespace kvfp4 {

// Cached-token count of sequence b, clamped to what its page-table row holds.
__device__ inline int clamped_len(const DecodeArgs& a, int b) {
  int L = a.seq_lens[b];
  const int cap = a.max_pages * a.g.T;
  if (L > cap) L = cap;
  if (L < 0) L = 0;
  return L;
}

__device__ inline int pages_of(const DecodeArgs& a, int b) {
  return (clamped_len(a, b) + a.g.T - 1) / a.g.T;
}

// floor(w P / nwg), in 32-bit arithmetic whenever P nwg fits (a 64-bit
// division is a long software sequence on the startup path)
__device__ inline long long range_begin(long long ptot, int w, int nwg) {
  if (ptot <= (long long)(0xFFFFFFFFu / (unsigned)nwg))
    return (long long)((unsigned)w * (unsigned)ptot / (unsigned)nwg);
  return (long long)w * ptot / nwg;
}

// Workgroups are dispatched to the 8 XCDs (each with its own L2) round
// robin: workgroup b runs on XCD b % 8.  The balanced split is numbered so
// that each XCD holds a contiguous block of it; neighbours in the split,
// which hold pages of the same sequences (its query rows, page-table lines
// and scale lines), then share an L2.  A bijection of [0, n).
constexpr int kXcds = 8;
__device__ inline int split_index(int b, int n) {
  const int x = b % kXcds, k = b / kXcds;
  const int q = n / kXcds, r = n % kXcds;
  return x * q + (x < r ? x : r) + k;
}

// Wave-uniform copies (values every lane already agrees on), so that the
// compiler keeps them in scalar registers and can build buffer resources
// and branch on them without per-lane loops.
__device__ inline int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ inline long long uniform(long long v) {
  unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(v & 0xFFFFFFFFu));
  unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)((unsigned long long)v >> 32));
  return (long long)(((unsigned long long)hi << 32) | lo);
}

struct BalancedRange {
  long long ptot;         // pages in the batch
  long long p_begin;      // this workgroup's pages [p_begin, p_end)
  long long p_end;
  int b_first;            // first sequence with pages in the range (batch if none)
  long long start_first;  // index of its first page in the concatenation
  int len0;               // lane l: clamped length of sequence l (l < 64)
};

// Wave-level inclusive prefix sum of an int over 64 lanes.
__device__ inline int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int t = __shfl_up(v, off);
    if (lane >= off) v += t;
  }
  return v;
}

// Computed by every wave on its own (no LDS, no barrier).  The first 64
// lengths are read once and kept (len0; most batches have at most 64
// sequences), so that the scan, the range search and the segment loop wait
// for one round of length loads.
__device__ inline void balanced_range(const DecodeArgs& a, int w, int nwg, BalancedRange& r) {
  const int lane = threadIdx.x & 63;
  r.len0 = lane < a.batch ? clamped_len(a, lane) : 0;
  const int np0 = (r.len0 + a.g.T - 1) / a.g.T;
  const int incl0 = wave_incl_scan(np0);
  long long tot = __shfl(incl0, 63);
  for (int base = 64; base < a.batch; base += 64) {
    int b = base + lane;
    int np = b < a.batch ? pages_of(a, b) : 0;
    tot += __shfl(wave_incl_scan(np), 63);
  }
  tot = uniform(tot);
  r.ptot = tot;
  r.p_begin = range_begin(tot, w, nwg);
  r.p_end = range_begin(tot, w + 1, nwg);
  r.b_first = a.batch;
  r.start_first = tot;
  if (r.p_begin >= r.p_end) return;
  long long run = 0;
  for (int base = 0; base < a.batch; base += 64) {
    int b = base + lane;
    int np = base == 0 ? np0 : (b < a.batch ? pages_of(a, b) : 0);
    int incl = base == 0 ? incl0 : wave_incl_scan(np);
    bool hit = np > 0 && run + incl > r.p_begin;
    unsigned long long m = __builtin_amdgcn_ballot_w64(hit);
    if (m) {
      int l0 = __builtin_ctzll(m);
      r.b_first = uniform(base + l0);
      r.start_first = uniform(run + __shfl(incl - np, l0));
      return;
    }
    run = uniform(run + __shfl(incl, 63));
  }
}

// Clamped length of sequence b (wave-uniform), from the lengths the range
// search kept when b < 64.
__device__ inline int seq_len(const DecodeArgs& a, const BalancedRange& r, int b) {
  return b < 64 ? __builtin_amdgcn_readlane(r.len0, b) : uniform(clamped_len(a, b));
}

// Records for the merge which workgroups hold sequence b's first and last
// pages (a single lane stores; the merge runs after this kernel ends).
__device__ inline void note_segment(const DecodeArgs& a, int w, int b, long long p_lo,
                                    long long p_hi, long long npages) {
  if (threadIdx.x == 0) {
    if (p_lo == 0) a.ws_idx[2 * b] = w;
    if (p_hi == npages) a.ws_idx[2 * b + 1] = w;
  }
}

// Workgroup 0 records the batch's page count (whether or not its range is empty).
__device__ inline void note_total(const DecodeArgs& a, int w, long long ptot) {
  if (w == 0 && threadIdx.x == 0) a.ws_idx[2 * a.batch] = (int32_t)ptot;
}

}  // namespace kvfp4
