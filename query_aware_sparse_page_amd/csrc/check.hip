// Device-side check of the input contents the host cannot see (sequence lengths, page ids, a
// selection): the caller's contract of every other entry point, verified on request.
//
// One block per sequence. Every read stays inside the arrays the descriptor sizes (page-table
// rows are read only below min(N_b, max_pages_per_seq)), so contents that break the contract are
// reported, never followed. Violations OR bits into *flags (sticky).
#include "kvsel_internal.h"

namespace kvsel {

constexpr int CHECK_THREADS = 256;

__global__ __launch_bounds__(CHECK_THREADS) void check_inputs_kernel(
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ seq_lens, int Hkv, int P,
    int maxp, int maxn, int Npp, const int32_t* __restrict__ page_fill,
    const int32_t* __restrict__ sel_idx, const int32_t* __restrict__ sel_cnt,
    int k, uint32_t* flags) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int L = seq_lens[b];
  uint32_t bad = 0;
  if (L < 0 || (long)L > (long)maxn * P) bad |= 1u;  // KVSEL_CHECK_SEQ_LEN (maxn <= maxp)
  const int N = L > 0 ? (int)min(((long)L + P - 1) / P, (long)maxp) : 0;
  for (int n = tid; n < N; n += CHECK_THREADS) {
    const int p = page_table[(size_t)b * maxp + n];
    if (p < 0 || p >= Npp) {
      bad |= 2u;  // KVSEL_CHECK_PAGE_ID
    } else if (page_fill && (page_fill[p] < 1 || page_fill[p] > P)) {
      bad |= 16u;  // KVSEL_CHECK_PAGE_FILL
    }
  }
  if (sel_idx) {
    const int lim = min(k, N);
    for (int j = 0; j < Hkv; ++j) {
      const int cnt = sel_cnt[(size_t)b * Hkv + j];
      if (cnt < 0 || cnt > lim) bad |= 4u;  // KVSEL_CHECK_SELECTION
      const int c = min(max(cnt, 0), k);
      const int32_t* row = sel_idx + ((size_t)b * Hkv + j) * k;
      for (int i = tid; i < c; i += CHECK_THREADS) {
        const int v = row[i];
        if (v < 0 || v >= N || (i > 0 && row[i - 1] >= v)) bad |= 4u;
      }
    }
  }
  if (bad) atomicOr(flags, bad);
}

hipError_t launch_check_inputs(const LaunchKV& kv, const int32_t* sel_idx, const int32_t* sel_cnt,
                               int k, uint32_t* flags, hipStream_t stream) {
  hipLaunchKernelGGL(check_inputs_kernel, dim3((unsigned)kv.B), dim3(CHECK_THREADS), 0, stream,
                     kv.page_table, kv.seq_lens, kv.Hkv, kv.P, kv.maxp, kv.maxn, kv.Npp, kv.page_fill, sel_idx, sel_cnt,
                     k, flags);
  return hipGetLastError();
}

}  // namespace kvsel
