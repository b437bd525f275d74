// Block-wide exact top-k by radix select over orderable 32-bit keys, shared by the selection
// kernels and the fused selection + attention kernel.
#pragma once

#include "kvsel_device.h"

namespace kvsel {

// LDS state of the radix select for a block of NT threads.
template <int NT>
struct RadixSmem {
  static constexpr int NW = NT / 64;
  // histogram copies: wave w counts into copy w % HC (one copy for up to 4 waves, where reading
  // and summing copies measured slower than the atomics they spread; 4 for larger blocks)
  static constexpr int HC = NW <= 4 ? 1 : 4;
  // three rotating sets of HC 256-bin histograms, as 64 uint4 (lane l reads bins 4l .. 4l+3)
  uint4 hist[3][HC][64];
  uint32_t wave_a[NW], wave_b[NW];      // scan totals
  uint32_t wave_min[NW], wave_max[NW];  // key range (own slots: read with no barrier after)
};

// Boundary bin of one radix pass, found by every wave on its own from the histogram totals
// (t = bins 4l .. 4l+3 of lane l): the bin b with above(b) < need <= above(b) + count(b), where
// above(b) counts the keys in larger bins. Returns the digit; need becomes need - above(b) and
// count the bin's total. The result is wave-uniform and identical in every wave.
__device__ __forceinline__ uint32_t boundary_bin(uint4 t, uint32_t& need, uint32_t& count) {
  const int lane = threadIdx.x & 63;
  const uint32_t incl = wave_scan_add(t.x + t.y + t.z + t.w);
  // keys above bins 4l+3, 4l+2, 4l+1, 4l (higher lanes hold the larger bins)
  const uint32_t a3 = __builtin_amdgcn_readlane(incl, 63) - incl;
  const uint32_t a2 = a3 + t.w, a1 = a2 + t.z, a0 = a1 + t.y;
  const bool h3 = a3 < need && need <= a2;
  const bool h2 = a2 < need && need <= a1;
  const bool h1 = a1 < need && need <= a0;
  const bool h0 = a0 < need && need <= a0 + t.x;
  const uint32_t sel = h3 ? 3u : h2 ? 2u : h1 ? 1u : 0u;
  const uint32_t above = h3 ? a3 : h2 ? a2 : h1 ? a1 : a0;
  const uint32_t cnt = h3 ? t.w : h2 ? t.z : h1 ? t.y : t.x;
  const int src = __builtin_ctzll(__ballot(h0 || h1 || h2 || h3));  // exactly one lane
  const uint32_t packed = __builtin_amdgcn_readlane((4u * lane + sel) | (above << 8), src);
  count = __builtin_amdgcn_readlane(cnt, src);
  need -= packed >> 8;
  return packed & 255u;
}

// Exclusive scan over the block of two counters (wave scans on DPP, one barrier for the wave
// totals); also returns nothing else: the block totals are not needed.
template <int NT>
__device__ __forceinline__ void block_exclusive_scan2(uint32_t a, uint32_t b, uint32_t& a_ex,
                                                      uint32_t& b_ex, RadixSmem<NT>& sm) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t ia = wave_scan_add(a), ib = wave_scan_add(b);
  if (lane == 63) {
    sm.wave_a[w] = ia;
    sm.wave_b[w] = ib;
  }
  __syncthreads();
  uint32_t ba = 0, bb = 0;
#pragma unroll
  for (int v = 0; v < NT / 64; ++v)
    if (v < w) {
      ba += sm.wave_a[v];
      bb += sm.wave_b[v];
    }
  a_ex = ba + ia - a;
  b_ex = bb + ib - b;
}

// Exact top-k of the N keys of one list, by the whole block, with the keys in registers: thread t
// holds the keys of indices t*C .. t*C + C - 1 (indices >= N are ignored). For every chosen index
// i, emit(pos, i, u) is called by the thread holding it (u = i - t*C), where pos < min(k, N) is
// its place in the ascending list of chosen indices; positions past min(k, N) are the caller's.
//
// Radix select over orderable keys, most significant digit first, starting below the bits all
// keys share (block min / max) and stopping as soon as the bucket holding the k-th largest key
// holds exactly the number of keys still needed. A pass is one predicated LDS atomic per key
// into histogram set pass % 3, one barrier, and a boundary search that every wave runs on its
// own over the totals (set pass + 1 is cleared before the barrier; its last readers, two passes
// back, all passed the previous barrier). The chosen set is {keys in buckets above the boundary
// bucket} plus the first `need` keys of the boundary bucket in index order (ties go to the lower
// index); one block scan over the per-thread index chunks gives every chosen index its place.
template <int NT, int C, class Emit>
__device__ void block_topk_regs(const uint32_t (&key)[C], int N, int k, RadixSmem<NT>& sm,
                                Emit emit) {
  constexpr int NW = NT / 64;
  constexpr int HC = RadixSmem<NT>::HC;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int i0 = tid * C;
  if (N <= k) {
#pragma unroll
    for (int u = 0; u < C; ++u)
      if (i0 + u < N) emit(i0 + u, i0 + u, u);
    return;
  }
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int u = 0; u < C; ++u) {
    if (i0 + u < N) {
      kmin = min(kmin, key[u]);
      kmax = max(kmax, key[u]);
    }
  }
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  for (int i = tid; i < HC * 64; i += NT) (&sm.hist[0][0][0])[i] = make_uint4(0, 0, 0, 0);
  if (lane == 0) {
    sm.wave_min[w] = kmin;
    sm.wave_max[w] = kmax;
  }
  __syncthreads();
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    kmin = min(kmin, sm.wave_min[v]);
    kmax = max(kmax, sm.wave_max[v]);
  }
  uint32_t prefix = kmax, mask = 0xffffffffu, need = (uint32_t)k;
  if (kmin != kmax) {
    const int top_bit = 31 - __clz((int)(kmin ^ kmax));
    mask = top_bit == 31 ? 0u : ~((2u << top_bit) - 1u);
    prefix = kmax & mask;
    for (int top = top_bit, pass = 0; top >= 0; top -= 8, ++pass) {
      const int cur = pass % 3, nxt = (pass + 1) % 3;
      const int shift = top >= 7 ? top - 7 : 0;
      const uint32_t dmask = (2u << (top - shift)) - 1u;
      for (int i = tid; i < HC * 64; i += NT) (&sm.hist[nxt][0][0])[i] = make_uint4(0, 0, 0, 0);
      uint32_t* h = (uint32_t*)&sm.hist[cur][w % HC][0];
#pragma unroll
      for (int u = 0; u < C; ++u) {
        if (i0 + u < N && (key[u] & mask) == prefix) atomicAdd(&h[(key[u] >> shift) & dmask], 1u);
      }
      __syncthreads();
      uint4 t = sm.hist[cur][0][lane];
#pragma unroll
      for (int c = 1; c < HC; ++c) {
        const uint4 x = sm.hist[cur][c][lane];
        t.x += x.x;
        t.y += x.y;
        t.z += x.z;
        t.w += x.w;
      }
      uint32_t count;
      const uint32_t digit = boundary_bin(t, need, count);
      prefix |= digit << shift;
      mask |= dmask << shift;
      if (count == need) break;  // the whole boundary bucket is taken
    }
  }
  // ---- compaction over the thread's contiguous indices ----
  uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
  for (int u = 0; u < C; ++u) {
    const uint32_t m = key[u] & mask;
    const bool ok = i0 + u < N;
    n_gt += ok && m > prefix;
    n_eq += ok && m == prefix;
  }
  uint32_t gt_ex, eq_ex;
  block_exclusive_scan2(n_gt, n_eq, gt_ex, eq_ex, sm);
  uint32_t pos = gt_ex + min(eq_ex, need);
  uint32_t eq_seen = eq_ex;
#pragma unroll
  for (int u = 0; u < C; ++u) {
    const int i = i0 + u;
    const uint32_t m = key[u] & mask;
    if (i < N) {
      const bool sel = m > prefix || (m == prefix && eq_seen < need);
      eq_seen += m == prefix;
      if (sel) {
        if (pos < (uint32_t)k) emit((int)pos, i, u);
        ++pos;
      }
    }
  }
}

}  // namespace kvsel
