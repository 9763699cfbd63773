// Balanced split-K over the pages of a whole batch (device side).
//
// The pages of all sequences, concatenated in batch order, form one list of
// P pages (sequence b contributes ceil(L_b / T) of them), with the pads
// described below between some sequences.  Workgroup w of nwg owns
// [floor(w P / nwg), floor((w+1) P / nwg)) of that list.  Every range is
// contiguous and ranges are monotone in w, so the (workgroup, sequence)
// pairs that overlap are indexed without collision by w + b: this is the
// partial slot the workgroup writes for that sequence.  Every workgroup
// computes the same ranges from seq_lens with the same integer arithmetic;
// the merge reads which workgroups held each sequence from the workspace.
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

// Segment pads.  A workgroup whose range holds the end of one sequence and
// the start of the next walks two segments: it starts twice (queries,
// page-table entries, the first tiles' wait with nothing else of its own in
// flight) and merges its streams twice.  Each sequence boundary that the
// plain split puts inside a range is therefore given a pad of a.seg_pad
// virtual pages (about 128 tokens' worth, set by the plan) in front of the
// next sequence's pages: the split is taken over real and pad pages
// together, so the workgroups around such a boundary take fewer real pages.
// Boundaries that fall on a range start cost no second segment and get no
// pad, so a batch whose sequences split evenly keeps the plain split.  The
// plan sets pads only for batches of at most 64 sequences, whose lengths the
// range search keeps in registers.

struct BalancedRange {
  long long ptot;         // length of the split: the batch's pages plus pads
  long long p_begin;      // this workgroup's share [p_begin, p_end) of it
  long long p_end;
  int b_first;            // first sequence with pages in the range (batch if none)
  long long start_first;  // its start in the split (its pad, if it has one)
  int len0;               // lane l: clamped length of sequence l (l < 64)
  int pad;                // pages of a pad
  unsigned long long padmask;  // bit b: sequence b's pages follow a pad
};

// Computed by every wave on its own (no LDS, no barrier).  The first 64
// lengths are read once and kept (len0; most batches have at most 64
// sequences), so that the scan, the range search and the segment loop wait
// for one round of length loads.
__device__ inline void balanced_range(const DecodeArgs& a, int w, int nwg, BalancedRange& r) {
  const int lane = threadIdx.x & 63;
  r.len0 = lane < a.batch ? clamped_len(a, lane) : 0;
  const int np0 = (r.len0 + a.g.T - 1) / a.g.T;
  const int incl0 = wave_incl_scan(np0);
  long long tot = __builtin_amdgcn_readlane(incl0, 63);
  for (int base = 64; base < a.batch; base += 64) {
    int b = base + lane;
    int np = b < a.batch ? pages_of(a, b) : 0;
    tot += __builtin_amdgcn_readlane(wave_incl_scan(np), 63);
  }
  tot = uniform(tot);
  // pads: sequence `lane` starts at page s of the plain split, and s starts
  // a range (s = floor(w P / nwg) for some w) exactly when a multiple of P
  // lies in [s nwg, s nwg + nwg): when (s nwg) mod P is 0 or above P - nwg.
  // The plan sets pads only where P nwg < 2^31, so 32-bit arithmetic holds;
  // the quotient comes from an fp32 estimate (within one of the truth, as
  // s nwg / P < nwg), corrected once each way.
  r.pad = a.seg_pad;
  r.padmask = 0;
  int vincl0 = incl0;  // end of the lane's sequence in the split, pads included
  if (r.pad > 0 && tot > nwg) {
    const unsigned P = (unsigned)tot, sn = (unsigned)(incl0 - np0) * (unsigned)nwg;
    const unsigned q = (unsigned)((float)sn * __builtin_amdgcn_rcpf((float)P));
    int rem = (int)(sn - q * P);
    rem += rem < 0 ? (int)P : 0;
    rem -= rem >= (int)P ? (int)P : 0;
    const bool padded = np0 > 0 && rem != 0 && rem <= (int)(P - (unsigned)nwg);
    r.padmask = __builtin_amdgcn_ballot_w64(padded);
    const unsigned long long upto = lane == 63 ? ~0ull : (2ull << lane) - 1ull;
    vincl0 = incl0 + r.pad * __builtin_popcountll(r.padmask & upto);
    tot = uniform(tot + (long long)r.pad * __builtin_popcountll(r.padmask));
  }
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
    int incl = base == 0 ? vincl0 : wave_incl_scan(np);
    bool hit = np > 0 && run + incl > r.p_begin;
    unsigned long long m = __builtin_amdgcn_ballot_w64(hit);
    if (m) {
      int l0 = __builtin_ctzll(m);
      const int padb = ((r.padmask >> l0) & 1) ? r.pad : 0;
      r.b_first = uniform(base + l0);
      r.start_first = uniform(run + __builtin_amdgcn_readlane(incl - np, l0) - padb);
      return;
    }
    run = uniform(run + __builtin_amdgcn_readlane(incl, 63));
  }
}

// Where sequence b's pages begin in the split, given where its share of the
// split begins (`start`: its pad, if it has one).
__device__ inline long long seq_first_page(const BalancedRange& r, int b, long long start) {
  return start + ((b < 64 && ((r.padmask >> b) & 1ull)) ? r.pad : 0);
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

// Workgroup 0 records the length of the split (whether or not its range is empty).
__device__ inline void note_total(const DecodeArgs& a, int w, long long ptot) {
  if (w == 0 && threadIdx.x == 0) a.ws_idx[2 * a.batch] = (int32_t)ptot;
}

}  // namespace kvfp4
