// Query-aware page scoring, top-k page selection and the speculative-reuse decision.
//
// score_kernel: one block per (page chunk, list), list = (sequence, KV head) varying fastest;
// each block scores 4 * PPW pages (score_block: summary loads, fp64 products, tail refresh).
//
// topk_kernel: one block per list. An exact radix select over orderable 32-bit score keys
// (8-bit digits, most significant first, starting below the bits all keys share, stopping once
// the boundary bucket is exactly what is still needed) finds the boundary; pages above it are
// taken and pages in the boundary bucket are taken in ascending page order (ties go to the lower
// index); a block scan gives each chosen page its slot in the ascending output. Its first wave
// evaluates the speculative-reuse decision.
//
// The two kernels are separate launches on purpose: a "last block of the list does the top-k"
// fusion needs a device-scope release / acquire per block, which on this GPU writes back and
// invalidates the XCD's L2 and measured slower than the second launch.
#include "kvsel_device.h"
#include "kvsel_internal.h"
#include "kvsel_score.h"
#include "kvsel_topk.h"

namespace kvsel {

constexpr int SEL_THREADS = 256;
constexpr int SEL_WAVES = SEL_THREADS / 64;
constexpr int SEL_LDS_KEYS = 8192;
constexpr int TOPK_BATCH = 8;  // independent score loads in flight per thread
constexpr int TOPK_WIDE_THREADS = 1024;  // top-k block for tables wider than TOPK_SMALL_PAGES
constexpr int TOPK_SMALL_PAGES = 4 * SEL_THREADS;

// Radix-select state plus an LDS copy of the keys (block_topk, which reads scores from memory).
template <int NT>
struct TopkSmem : RadixSmem<NT> {
  uint32_t keys[SEL_LDS_KEYS];
};

// Exact top-k of the N scores of one list, by the whole block; writes out[0..k) ascending
// (padded with -1) and, when `used` is non-null, the same list there too. `first` holds the
// caller's loads of sc[min(tid + u * NT, row - 1)] for u < TOPK_BATCH (issued before the
// sequence length is known, so they overlap its load).
//
// Radix select over orderable keys, most significant digit first, starting below the bits all
// keys share (block min / max) and stopping as soon as the bucket holding the k-th largest key
// holds exactly the number of keys still needed. Keys are loaded in batches of independent
// loads; histograms are per wave (no LDS atomic contention across waves); every scan and
// reduction runs on DPP. The chosen set is {keys in buckets above the boundary bucket} plus the
// first `need` keys of the boundary bucket in index order (ties to the lower page index); one
// block scan over per-thread contiguous index chunks gives every chosen page its output slot.
// This form reads the scores from memory (keeping them in LDS when they fit); lists whose keys
// fit in registers take block_topk_regs.
template <int NT>
__device__ void block_topk(const float* __restrict__ sc, const float* first, int N, int k,
                           int32_t* __restrict__ out, int32_t* __restrict__ used, TopkSmem<NT>& sm) {
  constexpr int BATCH = TOPK_BATCH;
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (N <= k) {
    for (int i = tid; i < k; i += NT) {
      const int v = i < N ? i : -1;
      out[i] = v;
      if (used) used[i] = v;
    }
    return;
  }
  const bool cached = N <= SEL_LDS_KEYS;
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  {
    float v[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) v[u] = first[u];
    for (int base = tid; base < N; base += NT * BATCH) {
      if (base != tid) {
#pragma unroll
        for (int u = 0; u < BATCH; ++u) v[u] = sc[min(base + u * NT, N - 1)];  // clamped
      }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int i = base + u * NT;
      if (i < N) {
        const uint32_t key = score_key(v[u]);
        if (cached) sm.keys[i] = key;
        kmin = min(kmin, key);
        kmax = max(kmax, key);
      }
    }
    }
  }
  constexpr int HC = TopkSmem<NT>::HC;
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
    // One barrier per pass: the counts go into set p % 3; after the barrier every wave reads the
    // totals and finds the boundary itself. Set (p + 1) % 3 is cleared before the barrier; its
    // last readers (pass p - 2) all passed the previous barrier.
    for (int top = top_bit, pass = 0; top >= 0; top -= 8, ++pass) {
      const int cur = pass % 3, nxt = (pass + 1) % 3;
      const int shift = top >= 7 ? top - 7 : 0;
      const uint32_t dmask = (2u << (top - shift)) - 1u;
      for (int i = tid; i < HC * 64; i += NT) (&sm.hist[nxt][0][0])[i] = make_uint4(0, 0, 0, 0);
      uint32_t* h = (uint32_t*)&sm.hist[cur][w % HC][0];
      for (int i = tid; i < N; i += NT) {
        const uint32_t u = cached ? sm.keys[i] : score_key(sc[i]);
        if ((u & mask) == prefix) atomicAdd(&h[(u >> shift) & dmask], 1u);
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
  // ---- compaction: thread t owns indices [t*C, t*C + C) ----
  const int C = (N + NT - 1) / NT;
  const int i0 = tid * C, i1 = min(N, i0 + C);
  uint32_t n_gt = 0, n_eq = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t u = (cached ? sm.keys[i] : score_key(sc[i])) & mask;
    n_gt += u > prefix;
    n_eq += u == prefix;
  }
  uint32_t gt_ex, eq_ex;
  block_exclusive_scan2(n_gt, n_eq, gt_ex, eq_ex, sm);
  uint32_t pos = gt_ex + min(eq_ex, need);
  uint32_t eq_seen = eq_ex;
  for (int i = i0; i < i1; ++i) {
    const uint32_t u = (cached ? sm.keys[i] : score_key(sc[i])) & mask;
    const bool sel = u > prefix || (u == prefix && eq_seen < need);
    eq_seen += u == prefix;
    if (sel) {
      if (pos < (uint32_t)k) {
        out[pos] = i;
        if (used) used[pos] = i;
      }
      ++pos;
    }
  }
}

template <typename T, int D, int G, int U, bool FP8>
__global__ __launch_bounds__(SEL_THREADS) void score_kernel(SelectArgs a) {
  // grid (Hkv, B, chunks): the indices need no division; KV heads vary fastest. Chunks run in
  // reverse order of z, so the blocks holding the sequences' last pages (the tail refresh, the
  // longest chain) are dispatched first.
  score_block<T, D, G, SEL_WAVES, U, FP8>(a, blockIdx.x, blockIdx.y, a.nchunks - 1 - blockIdx.z);
}

// block_topk_regs writing the ascending list to out (and used, when non-null), padded with -1.
template <int NT, int C>
__device__ void topk_to_list(const uint32_t (&key)[C], int N, int k, int32_t* __restrict__ out,
                             int32_t* __restrict__ used, RadixSmem<NT>& sm) {
  block_topk_regs<NT, C>(key, N, k, sm, [&](int pos, int i, int) {
    out[pos] = i;
    if (used) used[pos] = i;
  });
  for (int i = max(N, 0) + threadIdx.x; i < k; i += NT) {
    out[i] = -1;
    if (used) used[i] = -1;
  }
}

// Speculative-reuse decision of one list, by the block's first wave: the group-mean cosine
// similarity C of this step's and the previous step's queries; corrected = first step or C < tau.
// Every thread gets the decision.
template <typename T, int D, int G>
__device__ int reuse_decision(const SelectArgs& a, int list, int b, int j, int* s_corr) {
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (w == 0) {
    const double C = group_cosine<T, D>((const T*)a.q, (const T*)a.reuse.q_prev, a.Hkv, G, b, j);
    const int corr = (a.reuse.first_step || C < a.reuse.tau) ? 1 : 0;
    if (lane == 0) {
      *s_corr = corr;
      a.reuse.corrected[list] = (uint8_t)corr;
      if (a.reuse.similarity) a.reuse.similarity[list] = C;
    }
  }
  __syncthreads();
  return *s_corr;
}

// Selection outputs of one list once its keys are known (shared by both launch structures).
// topk(out, used) runs the block's selection.
template <int NT, class TopK>
__device__ void select_outputs(const SelectArgs& a, int list, int N, int corrected, bool reuse_on,
                               TopK topk) {
  const int tid = threadIdx.x;
  int32_t* used = (reuse_on && corrected) ? a.reuse.used_idx + (size_t)list * a.k : nullptr;
  topk(a.sel_idx + (size_t)list * a.k, used);
  const int cnt = N < a.k ? N : a.k;
  if (tid == 0) a.sel_cnt[list] = cnt;
  if (reuse_on) {
    if (corrected) {
      if (tid == 0) a.reuse.used_cnt[list] = cnt;
    } else {
      for (int i = tid; i < a.k; i += NT)
        a.reuse.used_idx[(size_t)list * a.k + i] = a.reuse.prev_idx[(size_t)list * a.k + i];
      if (tid == 0) a.reuse.used_cnt[list] = a.reuse.prev_cnt[list];
    }
  }
}

// Top-k of one list with C keys per thread in registers (C * NT >= row width). The score
// loads depend on the row width only, so they go out before the sequence length is known.
template <typename T, int D, int G, int NT, int C>
__device__ __forceinline__ void topk_regs(const SelectArgs& a, int list, int b, int j,
                                          TopkSmem<NT>& sm, int* s_corr) {
  const int tid = threadIdx.x;
  const float* sc = a.scores + (size_t)list * a.maxp;
  float v[C];
#pragma unroll
  for (int u = 0; u < C; ++u) v[u] = sc[min(tid * C + u, a.maxn - 1)];
  const int L = a.seq_lens[b];
  const int N = L > 0 ? min((L + a.P - 1) / a.P, a.maxn) : 0;
  const bool reuse_on = a.reuse.q_prev != nullptr;
  const int corrected = reuse_on ? reuse_decision<T, D, G>(a, list, b, j, s_corr) : 1;
  uint32_t key[C];
#pragma unroll
  for (int u = 0; u < C; ++u) key[u] = score_key(v[u]);
  select_outputs<NT>(a, list, N, corrected, reuse_on, [&](int32_t* out, int32_t* used) {
    topk_to_list<NT, C>(key, N, a.k, out, used, sm);
  });
}

// One block of NT threads per list: NT = 256 for tables of at most TOPK_SMALL_PAGES pages (up to 4
// keys per thread), 1024 for wider ones, so a 4096-page list is 4 keys per thread rather than 16
// (measured at 128K: 9.0 us per launch with 256 threads).
template <typename T, int D, int G, int NT>
__global__ __launch_bounds__(NT) void topk_kernel(SelectArgs a) {
  __shared__ TopkSmem<NT> sm;
  __shared__ int s_corr;
  const int tid = threadIdx.x;
  const int j = blockIdx.x, b = blockIdx.y;  // grid (Hkv, B)
  const int list = b * a.Hkv + j;
  const int cpt = (a.maxn + NT - 1) / NT;  // keys per thread
  if constexpr (NT == SEL_THREADS) {  // the host sends tables of <= 4 * NT pages here
    if (cpt <= 1) return topk_regs<T, D, G, NT, 1>(a, list, b, j, sm, &s_corr);
    if (cpt <= 2) return topk_regs<T, D, G, NT, 2>(a, list, b, j, sm, &s_corr);
    return topk_regs<T, D, G, NT, 4>(a, list, b, j, sm, &s_corr);
  } else {
    if (cpt <= 2) return topk_regs<T, D, G, NT, 2>(a, list, b, j, sm, &s_corr);
    if (cpt <= 4) return topk_regs<T, D, G, NT, 4>(a, list, b, j, sm, &s_corr);
    if (cpt <= 8) return topk_regs<T, D, G, NT, 8>(a, list, b, j, sm, &s_corr);
    // wider rows: scores re-read from memory by block_topk
    const float* sc = a.scores + (size_t)list * a.maxp;
    float first[TOPK_BATCH];
#pragma unroll
    for (int u = 0; u < TOPK_BATCH; ++u) first[u] = sc[min(tid + u * NT, a.maxn - 1)];
    const int L = a.seq_lens[b];
    const int N = L > 0 ? min((L + a.P - 1) / a.P, a.maxn) : 0;
    const bool reuse_on = a.reuse.q_prev != nullptr;
    const int corrected = reuse_on ? reuse_decision<T, D, G>(a, list, b, j, &s_corr) : 1;
    select_outputs<NT>(a, list, N, corrected, reuse_on, [&](int32_t* out, int32_t* used) {
      block_topk<NT>(sc, first, N, a.k, out, used, sm);
    });
  }
}

// ------------------------------------------------------------------------------------------
// One launch for lists of at most FUSED_MAX_PAGES pages: one 1024-thread block per list scores
// every page (keys straight into LDS) and then selects, so no score ever goes through memory
// and no second launch is needed. The summary loads (sequence-major rows) go out in batches of
// UNROLL pages per lane. Wave 0
// refreshes the tail page (when asked) and scores it from registers while the other waves score
// the rest.
// ------------------------------------------------------------------------------------------
constexpr int FUSED_THREADS = 1024;
constexpr int FUSED_MAX_PAGES = 2048;

template <typename T, int D, int G, bool FP8>
__global__ __launch_bounds__(FUSED_THREADS) void select_fused_kernel(SelectArgs a) {
  using M = row_map<T, D>;
  constexpr int VEC = M::VEC, LPR = M::LPR;
  constexpr int PPW = 64 / LPR;                     // pages per wave per iteration
  constexpr int PPI = (FUSED_THREADS / 64) * PPW;   // pages per block iteration
  // summary loads in flight per lane (8 at G 4 measured slower: 32 x 32K selection 29.3 against
  // 27.9 us)
  constexpr int UNROLL = G >= 4 ? 4 : 8;
  __shared__ TopkSmem<FUSED_THREADS> sm;
  __shared__ int s_corr;
  const int j = blockIdx.x, b = blockIdx.y;  // grid (Hkv, B)
  const int list = b * a.Hkv + j;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int P = a.P;
  const int L = a.seq_lens[b];
  const int N = L > 0 ? min((L + P - 1) / P, a.maxn) : 0;  // never past the live bound
  const int Hq = a.Hkv * G;
  const int c0 = (lane % LPR) * VEC;
  const bool refresh = a.refresh_tail && N > 0;
  const int n_end = refresh ? N - 1 : N;  // pages scored from stored summaries

  static_assert(FUSED_THREADS >= D, "one thread per channel");
  float qc[G];
  q_channel_load<T, D, G>((const T*)a.q + ((size_t)b * Hq + j * G) * D, qc);
  __shared__ double s_q[2][D];
  const QSums<VEC> qs = q_sums_shared<D, G, VEC>(qc, s_q, c0);

  // ---- wave 0: decode-time refresh of the tail page, scored from registers ----
  if (refresh && w == 0) {
    const int nt = N - 1;
    const int pt = min(max(a.page_table[(size_t)b * a.maxp + nt], 0), a.Npp - 1);
    float lo[VEC], hi[VEC];
    refresh_tile<T, D, FP8>(a, b, nt, pt, j, L - nt * P, lane, lo, hi);
    if (lane < LPR) {
      T* out = (T*)a.summ + ((size_t)list * a.maxp + nt) * 2 * D;
      store16(out + c0, pack<T>(lo));
      store16(out + D + c0, pack<T>(hi));
    }
    const double acc = page_score<VEC, LPR>(qs, lo, hi);
    if (lane == 0) {
      sm.keys[nt] = score_key((float)acc);
      if (a.write_scores) a.scores[(size_t)list * a.maxp + nt] = (float)acc;
    }
  }

  // ---- every other page ----
  for (int it0 = 0; it0 * PPI < n_end; it0 += UNROLL) {
    uint4 lo_raw[UNROLL], hi_raw[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int n = (it0 + u) * PPI + w * PPW + lane / LPR;
      const T* srow = (const T*)a.summ + ((size_t)list * a.maxp + min(n, n_end - 1)) * 2 * D + c0;
      lo_raw[u] = load16_nt(srow);
      hi_raw[u] = load16_nt(srow + D);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int n = (it0 + u) * PPI + w * PPW + lane / LPR;
      float lo[VEC], hi[VEC];
      unpack<T>(lo_raw[u], lo);
      unpack<T>(hi_raw[u], hi);
      const double acc = page_score<VEC, LPR>(qs, lo, hi);
      if (n < n_end && (lane % LPR) == 0) {
        sm.keys[n] = score_key((float)acc);
        if (a.write_scores) a.scores[(size_t)list * a.maxp + n] = (float)acc;
      }
    }
  }
  __syncthreads();
  const bool reuse_on = a.reuse.q_prev != nullptr;
  const int corrected = reuse_on ? reuse_decision<T, D, G>(a, list, b, j, &s_corr) : 1;
  static_assert(FUSED_MAX_PAGES == 2 * FUSED_THREADS, "one or two keys per thread");
  if (N <= FUSED_THREADS) {
    uint32_t key[1] = {sm.keys[tid]};
    select_outputs<FUSED_THREADS>(a, list, N, corrected, reuse_on, [&](int32_t* out, int32_t* used) {
      topk_to_list<FUSED_THREADS, 1>(key, N, a.k, out, used, sm);
    });
  } else {
    uint32_t key[2] = {sm.keys[2 * tid], sm.keys[2 * tid + 1]};
    select_outputs<FUSED_THREADS>(a, list, N, corrected, reuse_on, [&](int32_t* out, int32_t* used) {
      topk_to_list<FUSED_THREADS, 2>(key, N, a.k, out, used, sm);
    });
  }
}

template <typename T, int D>
static int pages_per_select_block() {
  return SEL_WAVES * (64 / row_map<T, D>::LPR);
}

int select_blocks_per_list(const LaunchKV& kv) {
  const int ppb = (kv.dtype == 0 ? (kv.D == 64 ? pages_per_select_block<float, 64>()
                                               : pages_per_select_block<float, 128>())
                                 : (kv.D == 64 ? pages_per_select_block<bf16_t, 64>()
                                               : pages_per_select_block<bf16_t, 128>())) *
                  score_unroll(kv.maxn, kv.B * kv.Hkv);
  return (kv.maxn + ppb - 1) / ppb;
}

template <typename T, int D, int G, bool FP8>
static hipError_t launch_select_t(const SelectArgs& a, hipStream_t stream) {
  // One block per list reads a whole list's summaries through one CU, so the one-launch form
  // pays only when there are enough lists to spread over the chip (measured on the bf16 path:
  // 8 lists of 1024 pages take 24.7 us in one launch against 10.2 us in two; 128 lists of up
  // to 1024 pages take 15.8 us against 18.6 us).
  if constexpr (G <= 4) {  // larger groups would spill at 1024 threads
    if (!a.scores_only && a.nlists >= SELECT_ONE_LAUNCH_MIN_LISTS && a.maxn <= FUSED_MAX_PAGES) {
      hipLaunchKernelGGL((select_fused_kernel<T, D, G, FP8>), dim3(a.Hkv, a.nlists / a.Hkv),
                         dim3(FUSED_THREADS), 0, stream, a);
      return hipGetLastError();
    }
  }
  const dim3 sgrid(a.Hkv, a.nlists / a.Hkv, a.nchunks);
  switch (score_unroll(a.maxn, a.nlists)) {
    case 1: hipLaunchKernelGGL((score_kernel<T, D, G, 1, FP8>), sgrid, dim3(SEL_THREADS), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((score_kernel<T, D, G, 2, FP8>), sgrid, dim3(SEL_THREADS), 0, stream, a); break;
    default: hipLaunchKernelGGL((score_kernel<T, D, G, 4, FP8>), sgrid, dim3(SEL_THREADS), 0, stream, a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.scores_only) return hipSuccess;
  if (a.maxn <= TOPK_SMALL_PAGES)
    hipLaunchKernelGGL((topk_kernel<T, D, G, SEL_THREADS>), dim3(a.Hkv, a.nlists / a.Hkv),
                       dim3(SEL_THREADS), 0, stream, a);
  else
    hipLaunchKernelGGL((topk_kernel<T, D, G, TOPK_WIDE_THREADS>), dim3(a.Hkv, a.nlists / a.Hkv),
                       dim3(TOPK_WIDE_THREADS), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D, bool FP8 = false>
static hipError_t launch_select_g(int G, const SelectArgs& a, hipStream_t stream) {
  switch (G) {
    case 1: return launch_select_t<T, D, 1, FP8>(a, stream);
    case 2: return launch_select_t<T, D, 2, FP8>(a, stream);
    case 4: return launch_select_t<T, D, 4, FP8>(a, stream);
    default: return launch_select_t<T, D, 8, FP8>(a, stream);
  }
}

// fp8 pools score bf16 summaries with a bf16 query; only the tail refresh reads the codes.
static hipError_t launch_select(const SelectArgs& a, const LaunchKV& kv, hipStream_t stream) {
  if (kv.dtype == 2) {
    if (kv.D == 64) return launch_select_g<bf16_t, 64, true>(kv.G, a, stream);
    return launch_select_g<bf16_t, 128, true>(kv.G, a, stream);
  }
  if (kv.dtype == 0) {
    if (kv.D == 64) return launch_select_g<float, 64>(kv.G, a, stream);
    return launch_select_g<float, 128>(kv.G, a, stream);
  }
  if (kv.D == 64) return launch_select_g<bf16_t, 64>(kv.G, a, stream);
  return launch_select_g<bf16_t, 128>(kv.G, a, stream);
}

SelectArgs select_args(const LaunchKV& kv, const RopeArgs& rope, void* summ, const void* q, int k,
                       int flags, int32_t* sel_idx, int32_t* sel_cnt, float* scores,
                       bool scores_requested, const ReuseArgs& reuse) {
  SelectArgs a;
  a.k_pool = kv.k_pool;
  a.summ = summ;
  a.q = q;
  a.page_table = kv.page_table;
  a.seq_lens = kv.seq_lens;
  a.Hkv = kv.Hkv;
  a.P = kv.P;
  a.maxp = kv.maxp;
  a.maxn = kv.maxn;
  a.Npp = kv.Npp;
  a.k = k;
  a.nlists = kv.B * kv.Hkv;
  a.nchunks = select_blocks_per_list(kv);
  a.refresh_tail = (flags & 1) ? 1 : 0;
  a.rope = rope;
  a.scores = scores;
  a.write_scores = scores_requested ? 1 : 0;
  a.sel_idx = sel_idx;
  a.sel_cnt = sel_cnt;
  a.reuse = reuse;
  a.scores_only = 0;
  a.k_scale = kv.k_scale;
  a.page_fill = kv.page_fill;
  return a;
}

hipError_t launch_score_topk(const LaunchKV& kv, const RopeArgs& rope, void* summ, const void* q,
                             int k, int flags, int32_t* sel_idx, int32_t* sel_cnt, float* scores,
                             bool scores_requested, const ReuseArgs& reuse, hipStream_t stream) {
  return launch_select(select_args(kv, rope, summ, q, k, flags, sel_idx, sel_cnt, scores,
                                   scores_requested, reuse),
                       kv, stream);
}

hipError_t launch_scores(const LaunchKV& kv, const RopeArgs& rope, void* summ, const void* q,
                         int flags, float* scores, hipStream_t stream) {
  SelectArgs a = select_args(kv, rope, summ, q, 1, flags, nullptr, nullptr, scores, true,
                             ReuseArgs{});
  a.scores_only = 1;
  return launch_select(a, kv, stream);
}

}  // namespace kvsel
