// Page scoring shared by the selection kernels (score_topk.hip) and the speculative-step launch
// that co-schedules scoring with attention (speculative.hip): the selection arguments, the
// min / max of one key tile (the tail refresh), the score of a chunk of pages by one block, and
// the group-mean query similarity of the speculative-reuse decision.
#pragma once

#include "kvsel_device.h"
#include "kvsel_fp8.h"
#include "kvsel_internal.h"

namespace kvsel {

struct SelectArgs {
  const void* k_pool;
  void* summ;
  const void* q;
  const int32_t* page_table;
  const int32_t* seq_lens;
  int Hkv, P, maxp, Npp, k, nlists, nchunks, refresh_tail, write_scores;
  int maxn;  // live pages at most (<= maxp, the row stride)
  int scores_only;  // launch the score kernel alone (the fused selection + attention call)
  RopeArgs rope;
  float* scores;
  int32_t* sel_idx;
  int32_t* sel_cnt;
  ReuseArgs reuse;
  const float* k_scale;  // fp8 pools: [Npp][Hkv] tile scales (the tail refresh)
  const int32_t* page_fill;  // [Npp] valid slots per physical page, or null (the tail refresh)
};

// Min / max of the valid rows (1 <= valid; more than P means the whole page; with page_fill, rows
// from page_fill[pt] on are excluded too, read after the row loads are issued) of one (page, KV
// head) tile of physical page pt, computed by one wave; rope_idx is its rotary page_row entry. On return every lane holds lo / hi of its
// channels [c0, c0 + VEC). The row loads are unconditional (rows past `valid` re-read the last
// valid row and are ignored), so they all go out at once; the page's rotary row is read after them.
template <typename T, int D>
__device__ __forceinline__ void tile_minmax(const T* tile, int valid, const int32_t* page_fill,
                                            int P, int lane, int pt, int rope_idx,
                                            const RopeArgs& rope, float* lo, float* hi) {
  valid = min(valid, P);  // a length past the page bound: every row of the last page counted
  using M = row_map<T, D>;
  constexpr int VEC = M::VEC, LPR = M::LPR, RPW = M::RPW;
  constexpr int MAX_LOADS = 32 / RPW;
  const int rg = lane / LPR;
  const int c0 = (lane % LPR) * VEC;
  uint4 raw[MAX_LOADS];
#pragma unroll
  for (int i = 0; i < MAX_LOADS; ++i) {
    const int s = rg + i * RPW;
    raw[i] = load16(tile + (size_t)min(s, valid - 1) * D + c0);
  }
  const int fill = page_fill ? page_fill[pt] : P;
  const int prow = rope.page_row ? rope.page_row[rope_idx] : -1;
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    lo[e] = __int_as_float(0x7f800000);
    hi[e] = __int_as_float(0xff800000);
  }
#pragma unroll
  for (int i = 0; i < MAX_LOADS; ++i) {
    const int s = rg + i * RPW;
    if (i * RPW >= P) break;
    float x[VEC];
    unpack<T>(raw[i], x);
    if (rope.page_row)
      rope_rotate_slice<T, D>(x, c0, prow < 0 ? -1 : prow + rope.row_step * s, rope.cos, rope.sin);
    if (s < valid && s < fill) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        lo[e] = fminf(lo[e], x[e]);
        hi[e] = fmaxf(hi[e], x[e]);
      }
    }
  }
#pragma unroll
  for (int m = LPR; m < 64; m <<= 1) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      lo[e] = fminf(lo[e], lane_xor_f32(lo[e], m));
      hi[e] = fmaxf(hi[e], lane_xor_f32(hi[e], m));
    }
  }
}

// The tail refresh's rebuild of the (physical page pt, KV head j) tile's summary by one wave: the
// min / max of its valid rows, rotated first when the rotary gather is on (f32 / bf16 pools), or
// scaled and rounded outward to bf16 (fp8 pools).
template <typename T, int D, bool FP8>
__device__ __forceinline__ void refresh_tile(const SelectArgs& a, int b, int n, int pt, int j,
                                             int valid, int lane, float* lo, float* hi) {
  const size_t t = (size_t)pt * a.Hkv + j;
  if constexpr (FP8)
    tile_minmax_fp8<D>((const uint8_t*)a.k_pool + t * a.P * D, valid, a.page_fill, pt, a.P, lane,
                       a.k_scale[t], lo, hi);
  else
    tile_minmax<T, D>((const T*)a.k_pool + t * a.P * D, valid, a.page_fill, a.P, lane, pt,
                      rope_row_index(a.rope, b, n, pt), a.rope, lo, hi);
}

// Scores of chunk `chunk` (WAVES * U * 64 / LPR consecutive pages) of list (sequence b, KV head
// j), by one block of WAVES waves: LPR lanes read a page's lo and hi rows as 16-byte slices
// (sequence-major summaries: one contiguous run per wave and unroll step), multiply by the group's
// query slice in fp64 (a bf16 x bf16 or fp32 x fp32 product is exact in fp64), take q*hi for
// q >= 0 and q*lo otherwise, and fold the LPR lanes; one fp64 -> fp32 rounding per score. Each
// lane group scores U pages (U > 1 for wide tables: fewer blocks, more loads in flight per lane).
// With the tail refresh on, the wave holding the sequence's last page first rebuilds that page's
// summary from the key pool, writes it, and scores it from the fresh values.
template <typename T, int D, int G, int WAVES, int U = 1, bool FP8 = false>
__device__ __forceinline__ void score_block(const SelectArgs& a, int j, int b, int chunk) {
  using M = row_map<T, D>;
  constexpr int VEC = M::VEC, LPR = M::LPR;
  constexpr int PPW = 64 / LPR;          // pages per wave and unroll step
  constexpr int PPB = WAVES * PPW * U;   // pages per block

  const int list = b * a.Hkv + j;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int P = a.P;
  const int wn0 = chunk * PPB + w * PPW * U;  // first page of this wave
  const int Hq = a.Hkv * G;
  const T* q = (const T*)a.q;
  const int c0 = (lane % LPR) * VEC;
  const int rgl = lane / LPR;  // the lane's row group: page wn0 + u * PPW + rgl at step u

  // ---- loads first (unconditional, clamped addresses), all in one round: the page ids (used
  // only for the tail refresh), q slice, summary rows (sequence-major, so no page-table hop) and
  // the sequence length ----
  // the page ids first: the wave that refreshes the tail page waits for them alone (loads
  // complete in issue order) and sends its key-tile loads while the summary rows are in flight
  // (entries past the sequence may hold anything and are clamped into the pool, never used)
  int pt_raw[U];
#pragma unroll
  for (int u = 0; u < U; ++u)  // indices from the row width only: no wait for seq_lens
    pt_raw[u] = a.page_table[(size_t)b * a.maxp + min(wn0 + u * PPW + rgl, a.maxn - 1)];
  uint4 qraw[G];
#pragma unroll
  for (int g = 0; g < G; ++g) qraw[g] = load16(q + ((size_t)b * Hq + j * G + g) * D + c0);
  uint4 lo_raw[U], hi_raw[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int nc = min(wn0 + u * PPW + rgl, a.maxn - 1);
    const T* srow = (const T*)a.summ + ((size_t)list * a.maxp + nc) * 2 * D + c0;
    lo_raw[u] = load16(srow);
    hi_raw[u] = load16(srow + D);
  }
  __builtin_amdgcn_sched_barrier(0);
  const int L = a.seq_lens[b];
  const int N = L > 0 ? min((L + P - 1) / P, a.maxn) : 0;  // never past the live bound

  // ---- decode-time refresh of the tail page's summary, by the wave that scores that page: the
  // page id is already in its lanes, so the key tile loads go out one hop after the page table,
  // alongside the summary loads, and no other wave waits ----
  const int nt = N - 1;
  const bool tail = a.refresh_tail && N > 0 && nt >= wn0 && nt < wn0 + PPW * U;  // wave-uniform
  const int t_off = nt - wn0;
  const int ut = tail ? t_off / PPW : -1, rg = t_off % PPW;  // its unroll step and row group
  float flo[VEC], fhi[VEC];
  if (tail) {
    int pt = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {  // scalar selects (a uniform index into pt_raw would spill it)
      const int x = __builtin_amdgcn_readlane(pt_raw[u], rg * LPR);
      pt = u == ut ? x : pt;
    }
    pt = min(max(pt, 0), a.Npp - 1);
    refresh_tile<T, D, FP8>(a, b, nt, pt, j, L - nt * P, lane, flo, fhi);
    if (lane < LPR) {
      T* out = (T*)a.summ + ((size_t)list * a.maxp + nt) * 2 * D;
      store16(out + c0, pack<T>(flo));
      store16(out + D + c0, pack<T>(fhi));
    }
  }

  // ---- scores of this wave's pages ----
  double qd[G][VEC];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float f[VEC];
    unpack<T>(qraw[g], f);
#pragma unroll
    for (int e = 0; e < VEC; ++e) qd[g][e] = (double)f[e];
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float lo[VEC], hi[VEC];
    unpack<T>(lo_raw[u], lo);
    unpack<T>(hi_raw[u], hi);
    if (u == ut && rgl == rg) {  // the stale rows loaded above are replaced by the fresh ones
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        lo[e] = flo[e];
        hi[e] = fhi[e];
      }
    }
    double acc = 0.0;
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const double x = (double)(qd[g][e] >= 0.0 ? hi[e] : lo[e]);
        acc = fma(qd[g][e], x, acc);
      }
    }
    acc = seg_sum_f64<LPR>(acc);
    const int n = wn0 + u * PPW + rgl;
    if (n < N && (lane % LPR) == 0) a.scores[(size_t)list * a.maxp + n] = (float)acc;
  }
}

// Unroll (pages per lane group) of the score kernel for a live page bound: long lists take fewer,
// fuller blocks.
inline int score_unroll(int maxn) { return maxn <= 1024 ? 1 : maxn <= 2048 ? 2 : 4; }

// Group-mean cosine similarity of this step's and the previous step's queries for KV head j of
// sequence b, by one wave, in fp64: for each of the G heads, dot / (|q| |q_prev|) with the
// channel sums taken lane-strided and folded across the wave; then the mean over the group.
// Every lane returns the same value, and every caller gets the same bits.
template <typename T, int D>
__device__ __forceinline__ double group_cosine(const T* q, const T* q_prev, int Hkv, int G, int b,
                                               int j) {
  const int lane = threadIdx.x & 63;
  const int Hq = Hkv * G;
  double csum = 0.0;
  for (int g = 0; g < G; ++g) {
    const size_t row = ((size_t)b * Hq + j * G + g) * D;
    double dot = 0.0, na = 0.0, nb = 0.0;
    for (int d = lane; d < D; d += 64) {
      const double xv = (double)load_elem<T>(q + row, d), yv = (double)load_elem<T>(q_prev + row, d);
      dot = fma(xv, yv, dot);
      na = fma(xv, xv, na);
      nb = fma(yv, yv, nb);
    }
    dot = seg_sum_f64<64>(dot);
    na = seg_sum_f64<64>(na);
    nb = seg_sum_f64<64>(nb);
    csum += dot / (sqrt(na) * sqrt(nb));
  }
  return csum / G;
}

// Host: the selection arguments of one call (score_topk.hip).
SelectArgs select_args(const LaunchKV& kv, const RopeArgs& rope, void* summ, const void* q, int k,
                       int flags, int32_t* sel_idx, int32_t* sel_cnt, float* scores,
                       bool scores_requested, const ReuseArgs& reuse);

}  // namespace kvsel
