// Page-list order for the codec calls (a scheduling aid; the results of the
// codec do not depend on it).
//
// The codec kernels take their pages in list order, so the workgroups that
// run at once work on neighbouring list entries.  When the list names the
// pool's slots in a random order, those workgroups touch pages scattered
// over the pool; with the same list sorted by slot they touch neighbouring
// pages, which the memory system streams faster.  This kernel sorts a list
// of (key, other) slot pairs by key: ascending as unsigned 32-bit values,
// equal keys in input order.
//
// One workgroup of 1024 threads sorts a run of up to kSortRun entries.
//  - Distinct keys in [0, kSortSlots) (a page list naming each slot once,
//    the usual case): each entry is placed at its key in an LDS table, and
//    the occupied places are read out in order (a counting sort: a few
//    passes over the table, whatever the order of the list).
//  - Otherwise a bitonic network over 64-bit words (key in the high half,
//    the entry's index in the low half) in LDS: the words are distinct, so
//    the order is total, equal keys stay in index order and every run of
//    the kernel gives the same result.
// A list longer than kSortRun is sorted in consecutive runs, one workgroup
// each.
#include "common.hpp"

namespace kvfp4 {

namespace {

constexpr int kSortThreads = 1024;
constexpr int kSortWaves = kSortThreads / 64;
constexpr int kSortRun = 16384;    // entries of a run (the network: 128 KiB of LDS)
constexpr int kSortSlots = 32768;  // keys the table holds (128 KiB of LDS)
constexpr size_t kSortLds = (size_t)kSortRun * 8 > (size_t)kSortSlots * 4
                                ? (size_t)kSortRun * 8 : (size_t)kSortSlots * 4;

__global__ __launch_bounds__(kSortThreads) void sort_pages_kernel(
    const int32_t* __restrict__ key, const int32_t* __restrict__ other, int n,
    int32_t* __restrict__ key_out, int32_t* __restrict__ other_out) {
  extern __shared__ unsigned long long word[];  // the network, or the table
  int* table = reinterpret_cast<int*>(word);
  __shared__ int s_max, s_bad, s_wave[kSortWaves];
  const int tid = threadIdx.x;
  const int base = blockIdx.x * kSortRun;
  const int m = n - base < kSortRun ? n - base : kSortRun;

  // Distinct keys in [0, kSortSlots)?  The largest key bounds the table.
  if (tid == 0) {
    s_max = 0;
    s_bad = 0;
  }
  __syncthreads();
  int kmax = 0;
  bool bad = false;
  for (int i = tid; i < m; i += kSortThreads) {
    const int k = key[base + i];
    bad |= k < 0 || k >= kSortSlots;
    kmax = k > kmax ? k : kmax;
  }
  // one LDS atomic per wave (a thousand on one address serialize)
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const int o = __shfl_xor(kmax, off);
    kmax = o > kmax ? o : kmax;
  }
  const bool any_bad = __builtin_amdgcn_ballot_w64(bad) != 0;
  if ((tid & 63) == 0) {
    if (any_bad) atomicOr(&s_bad, 1);
    atomicMax(&s_max, kmax);
  }
  __syncthreads();
  if (s_bad == 0) {
    const int slots = s_max + 1;
    for (int i = tid; i < slots; i += kSortThreads) table[i] = -1;
    __syncthreads();
    for (int i = tid; i < m; i += kSortThreads)
      if (atomicExch(&table[key[base + i]], i) != -1) atomicOr(&s_bad, 2);  // repeated key
    __syncthreads();
  }
  if (s_bad == 0) {
    // Read the table out in order: wave w owns places [w R / 16, (w+1) R / 16)
    // and walks them 64 at a time; a ballot over the occupied places gives
    // each lane its output position, so consecutive lanes write consecutive
    // entries.  One pass counts, a scan over the waves places them, a
    // second pass writes.
    const int slots = s_max + 1;
    const int lane = tid & 63, wave = tid >> 6;
    const int q0 = (int)((long long)wave * slots / kSortWaves);
    const int q1 = (int)((long long)(wave + 1) * slots / kSortWaves);
    int count = 0;
    for (int q = q0; q < q1; q += 64) {
      const bool hit = q + lane < q1 && table[q + lane] >= 0;
      count += __builtin_popcountll(__builtin_amdgcn_ballot_w64(hit));
    }
    if (lane == 0) s_wave[wave] = count;
    __syncthreads();
    int o = base;
    for (int w = 0; w < wave; ++w) o += s_wave[w];
    for (int q = q0; q < q1; q += 64) {
      const int i = q + lane < q1 ? table[q + lane] : -1;
      const unsigned long long hits = __builtin_amdgcn_ballot_w64(i >= 0);
      if (i >= 0) {
        const int at = o + (int)__builtin_popcountll(hits & ((1ull << lane) - 1ull));
        key_out[at] = q + lane;
        if (other_out) other_out[at] = other[base + i];
      }
      o += (int)__builtin_popcountll(hits);
    }
    return;
  }

  int len = 1;  // the network's size: a power of two >= m
  while (len < m) len <<= 1;
  for (int i = tid; i < len; i += kSortThreads)
    word[i] = i < m ? ((unsigned long long)(uint32_t)key[base + i] << 32) | (uint32_t)i
                    : ~0ull;  // padding sorts last
  __syncthreads();
  // stage `size`: sorted runs of size/2 become sorted runs of size,
  // ascending where bit `size` of the index is clear; pass `stride`
  // compares index lo (bit `stride` clear) with lo + stride
  for (int size = 2; size <= len; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = tid; t < len / 2; t += kSortThreads) {
        const int lo = 2 * t - (t & (stride - 1));
        const int hi = lo + stride;
        const bool ascending = (lo & size) == 0;
        const unsigned long long a = word[lo], b = word[hi];
        if ((a > b) == ascending) {
          word[lo] = b;
          word[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < m; i += kSortThreads) {
    const int from = base + (int)(uint32_t)word[i];
    key_out[base + i] = key[from];
    if (other_out) other_out[base + i] = other[from];
  }
}

std::atomic<unsigned long long> sort_lds_set{0};

}  // namespace

hipError_t launch_sort_pages(const int32_t* key, const int32_t* other, int num_pages,
                             int32_t* key_out, int32_t* other_out, hipStream_t stream) {
  if (num_pages == 0) return hipSuccess;
  hipError_t e = allow_lds_once(sort_lds_set, (const void*)sort_pages_kernel, kSortLds);
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)((num_pages + kSortRun - 1) / kSortRun);
  hipLaunchKernelGGL(sort_pages_kernel, dim3(grid), dim3(kSortThreads), kSortLds, stream, key,
                     other, num_pages, key_out, other_out);
  return hipGetLastError();
}

}  // namespace kvfp4
