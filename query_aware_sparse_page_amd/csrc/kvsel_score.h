// Page scoring shared by the selection kernels (score_topk.hip) and the speculative-step launch
// that co-schedules scoring with attention (speculative.hip): the selection arguments, the
// min / max of one key tile (the tail refresh), the score of a chunk of pages by one block, and
// the group-mean query similarity of the speculative-reuse decision.
#pragma once

#include <type_traits>

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

// ---- min / max of one key tile (the summary build and its tail refresh) ----

// One wave's share of the rows of one (page, KV head) tile: wave wv of the NW waves that share the
// tile takes rows wv * RPW + rg + i * NW * RPW (rg the lane's row group). Row indices at or past
// `valid` (1 <= valid <= P) are clamped to valid - 1, so every load reads -- and, with the rotary
// gather, rotates -- a valid row and a fold over all of them needs no guard; loads past the page
// (P = 16) repeat the wave's first row. fp8 pools (FP8): 8 codes per lane and row (bf16's layout).
template <typename T, int D, int NW, bool FP8>
struct TileRows {
  using M = row_map<T, D>;
  static constexpr int VEC = M::VEC, LPR = M::LPR, RPW = M::RPW;
  static constexpr int STRIDE = NW * RPW;                 // rows between a lane's loads
  static constexpr int NL = (32 + STRIDE - 1) / STRIDE;   // loads per lane: a page has <= 32 rows
  using Raw = std::conditional_t<FP8, uint2, uint4>;
  Raw raw[NL];
  int first, last, P;  // the lane's first row, the last valid row, the page size

  // Row of load i (recomputed where needed: the kernels that hold a whole block's work in
  // registers cannot spare one per load).
  __device__ __forceinline__ int row(int i) const {
    return min(i * STRIDE < P ? first + i * STRIDE : first, last);
  }

  __device__ __forceinline__ void load(const void* tile, int valid, int P_, int lane, int wv) {
    first = wv * RPW + lane / LPR;
    last = valid - 1;
    P = P_;
    const int c0 = (lane % LPR) * VEC;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      if constexpr (FP8)
        raw[i] = load8_nt((const uint8_t*)tile + (size_t)row(i) * D + c0);
      else
        raw[i] = load16_nt((const T*)tile + (size_t)row(i) * D + c0);
    }
  }

  // Row i's slice as fp32 (unpacked; fp8 codes decoded, unscaled).
  __device__ __forceinline__ void decode(int i, float* x) const {
    if constexpr (FP8)
      fp8x8_to_f32(raw[i], x);
    else
      unpack<T>(raw[i], x);
  }

  // Min / max over the lane's rows. Without a guard or rotation every row folds in, starting from
  // the first, so the compiler may pair rows into three-operand min / max. With page_fill (GUARD)
  // or the rotary gather (ROPE), lo / hi start at +inf / -inf and take one row at a time, rows at
  // or past `valid` or `fill` skipped: a rotated row uses its own position (prow: the page's first
  // rotary row, -1 for none), and each row's cos / sin loads stay live for that row only.
  template <bool ROPE, bool GUARD>
  __device__ __forceinline__ void fold(int c0, int valid, int fill, int prow,
                                       const RopeArgs& rope, float* lo, float* hi) const {
    if constexpr (!ROPE && !GUARD) {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        float x[VEC];
        decode(i, x);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          lo[e] = i == 0 ? x[e] : tmin(lo[e], x[e]);
          hi[e] = i == 0 ? x[e] : tmax(hi[e], x[e]);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        lo[e] = __int_as_float(0x7f800000);
        hi[e] = __int_as_float(0xff800000);
      }
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        if (i * STRIDE >= P) break;
        const int s = first + i * STRIDE;  // the row itself (loads past `valid` were clamped)
        float x[VEC];
        decode(i, x);
        if constexpr (ROPE)  // every lane takes part in the partner exchange
          rope_rotate_slice<T, D>(x, c0, prow < 0 ? -1 : prow + rope.row_step * s, rope.cos,
                                  rope.sin);
        if (s < valid && s < fill) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            lo[e] = tmin(lo[e], x[e]);
            hi[e] = tmax(hi[e], x[e]);
          }
        }
      }
    }
  }
};

// Min / max of lane's channels [c0, c0 + VEC) over its rows of wave wv's share (of NW) of the
// valid rows of one tile of physical page pt (1 <= valid; more than P means the whole page; with
// page_fill, rows from page_fill[pt] on are excluded too, read after the row loads are issued);
// rope_idx is the page's rotary page_row entry (f32 / bf16 pools). Not folded across lanes.
// start() issues every load, finish() folds: work that needs none of the tile can run between.
template <typename T, int D, int NW, bool FP8>
struct TileMinMax {
  TileRows<T, D, NW, FP8> r;
  int c0, valid, fill, prow;
  bool rot, guard;

  __device__ __forceinline__ void start(const void* tile, int valid_, const int32_t* page_fill,
                                        int P, int lane, int wv, int pt, int rope_idx,
                                        const RopeArgs& rope) {
    valid = min(valid_, P);
    r.load(tile, valid, P, lane, wv);
    c0 = (lane % row_map<T, D>::LPR) * row_map<T, D>::VEC;
    rot = !FP8 && rope.page_row != nullptr;
    prow = rot ? rope.page_row[rope_idx] : -1;
    guard = page_fill != nullptr;
    fill = guard ? page_fill[pt] : P;
  }

  __device__ __forceinline__ void finish(const RopeArgs& rope, float* lo, float* hi) const {
    if (rot)
      r.template fold<!FP8, true>(c0, valid, fill, prow, rope, lo, hi);
    else if (guard)
      r.template fold<false, true>(c0, valid, fill, prow, rope, lo, hi);
    else
      r.template fold<false, false>(c0, valid, fill, prow, rope, lo, hi);
  }
};

template <typename T, int D, int NW, bool FP8>
__device__ __forceinline__ void tile_rows_minmax(const void* tile, int valid,
                                                 const int32_t* page_fill, int P, int lane, int wv,
                                                 int pt, int rope_idx, const RopeArgs& rope,
                                                 float* lo, float* hi) {
  TileMinMax<T, D, NW, FP8> m;
  m.start(tile, valid, page_fill, P, lane, wv, pt, rope_idx, rope);
  m.finish(rope, lo, hi);
}

// lo / hi folded over the lanes that share a channel slice (lane ^ LPR, ..., lane ^ 32): every
// lane ends with the min / max of its channels.
template <int LPR, int VEC>
__device__ __forceinline__ void fold_lanes(float* lo, float* hi) {
#pragma unroll
  for (int m = LPR; m < 64; m <<= 1) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      lo[e] = tmin(lo[e], lane_xor_f32(lo[e], m));
      hi[e] = tmax(hi[e], lane_xor_f32(hi[e], m));
    }
  }
}

// Values a lane keeps after fold_lanes_scatter: one halving per lane swap (m = 16 and m = 32).
template <int LPR, int VEC>
constexpr int scatter_kept() { return LPR <= 16 ? VEC / 4 : VEC / 2; }

// The fold of fold_lanes as a reduce-scatter: at m = 16 and m = 32 one lane swap (gfx950 permlane16 /
// permlane32 swap of lo[i] and lo[i + h]) moves two values at once, and the min of the swapped pair
// leaves lo[i]'s result in one half of the lanes and lo[i + h]'s in the other; each step halves
// what a lane holds, at one swap and one min / max per pair. A smaller xor (8 lanes per row) folds
// in full first. On return lo / hi[0, K) (K = scatter_kept) are the results for channels
// c0 + off + [0, K); the return value is off.
template <int LPR, int VEC>
__device__ __forceinline__ int fold_lanes_scatter(float* lo, float* hi) {
  static_assert(LPR >= 8 && LPR <= 32, "lanes per row");
#pragma unroll
  for (int m = LPR; m < 16; m <<= 1) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      lo[e] = tmin(lo[e], lane_xor_f32(lo[e], m));
      hi[e] = tmax(hi[e], lane_xor_f32(hi[e], m));
    }
  }
  const int lane = threadIdx.x & 63;
  int n = VEC, off = 0;
  if constexpr (LPR <= 16) {  // rows of 16 lanes: odd rows take lo[i + h]
    const int h = n / 2;
#pragma unroll
    for (int i = 0; i < h; ++i) {
      auto rl = __builtin_amdgcn_permlane16_swap(__float_as_uint(lo[i]), __float_as_uint(lo[i + h]), false, false);
      auto rh = __builtin_amdgcn_permlane16_swap(__float_as_uint(hi[i]), __float_as_uint(hi[i + h]), false, false);
      lo[i] = tmin(__uint_as_float(rl[0]), __uint_as_float(rl[1]));
      hi[i] = tmax(__uint_as_float(rh[0]), __uint_as_float(rh[1]));
    }
    off += (lane & 16) ? h : 0;
    n = h;
  }
  {  // halves of 32 lanes: the upper half takes lo[i + h]
    const int h = n / 2;
#pragma unroll
    for (int i = 0; i < h; ++i) {
      auto rl = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo[i]), __float_as_uint(lo[i + h]), false, false);
      auto rh = __builtin_amdgcn_permlane32_swap(__float_as_uint(hi[i]), __float_as_uint(hi[i + h]), false, false);
      lo[i] = tmin(__uint_as_float(rl[0]), __uint_as_float(rl[1]));
      hi[i] = tmax(__uint_as_float(rh[0]), __uint_as_float(rh[1]));
    }
    off += (lane & 32) ? h : 0;
  }
  return off;
}

// fp8 tile extremes (codes' values) times the tile's scale, rounded outward to bf16; a code's
// value times an fp32 scale is exact in fp64.
template <int VEC>
__device__ __forceinline__ void fp8_scale_outward(float scale, float* lo, float* hi) {
  const double sd = (double)scale;
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    lo[e] = __uint_as_float(f64_to_bf16_directed<false>((double)lo[e] * sd) << 16);
    hi[e] = __uint_as_float(f64_to_bf16_directed<true>((double)hi[e] * sd) << 16);
  }
}

// Min / max of the valid rows of one (page, KV head) tile, computed by one wave: on return every
// lane holds lo / hi of its channels [c0, c0 + VEC), rotated first when the rotary gather is on.
template <typename T, int D>
__device__ __forceinline__ void tile_minmax(const T* tile, int valid, const int32_t* page_fill,
                                            int P, int lane, int pt, int rope_idx,
                                            const RopeArgs& rope, float* lo, float* hi) {
  tile_rows_minmax<T, D, 1, false>(tile, valid, page_fill, P, lane, 0, pt, rope_idx, rope, lo, hi);
  fold_lanes<row_map<T, D>::LPR, row_map<T, D>::VEC>(lo, hi);
}

// The same for an fp8 tile (bf16's lane layout, 8 channels per lane), times the tile's scale and
// rounded outward to bf16: every lane holds bf16 values in fp32.
template <int D>
__device__ __forceinline__ void tile_minmax_fp8(const uint8_t* tile, int valid,
                                                const int32_t* page_fill, int pt, int P, int lane,
                                                float scale, float* lo, float* hi) {
  tile_rows_minmax<bf16_t, D, 1, true>(tile, valid, page_fill, P, lane, 0, pt, 0, RopeArgs{}, lo,
                                       hi);
  fold_lanes<row_map<bf16_t, D>::LPR, row_map<bf16_t, D>::VEC>(lo, hi);
  fp8_scale_outward<row_map<bf16_t, D>::VEC>(scale, lo, hi);
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

// The group's query folded per channel, in fp64: qp[e] sums the G heads' non-negative values of
// channel e and qn[e] the negative ones (exact for bf16 queries, and for fp32 queries whose G
// values span at most 29 binary orders). Then the sum over the group of q*hi for q >= 0 and q*lo
// otherwise is, per channel, qp*hi + qn*lo: the same sum with two products per channel and page
// instead of 2G selects and G products, and no per-page work on the query. A lane holds the sums
// of its VEC channels.
template <int VEC>
struct QSums {
  double qp[VEC], qn[VEC];
};

// The channel sums are formed once per block: thread d < D loads channel d of the G heads with the
// block's first loads (q_channel_load), folds it in head order into LDS, and after one barrier
// every lane reads the sums of its VEC channels (q_sums_shared; block-uniform, blocks of at least
// D threads). q_sums_read re-reads them later from the same LDS.
template <typename T, int D, int G>
__device__ __forceinline__ void q_channel_load(const T* qrow, float (&qc)[G]) {
  const int d = min((int)threadIdx.x, D - 1);
#pragma unroll
  for (int g = 0; g < G; ++g) qc[g] = load_elem<T>(qrow, (size_t)g * D + d);
}

// LDS slot of channel c's sum: channel pairs (2i, 2i + 1) of the D / VEC lane slices side by side,
// so the lanes of a row group read their pair i from consecutive 16-byte slots (a lane's VEC
// channels in one run would put the lanes 8 * VEC bytes apart, on the same banks).
template <int D, int VEC>
__device__ __forceinline__ int q_sum_slot(int c) {
  static_assert(VEC % 2 == 0, "channel pairs");
  constexpr int LPR = D / VEC;
  return (((c % VEC) >> 1) * LPR + c / VEC) * 2 + (c & 1);
}

template <int D, int VEC>
__device__ __forceinline__ QSums<VEC> q_sums_read(const double (&s_q)[2][D], int c0) {
  QSums<VEC> r;
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    r.qp[e] = s_q[0][q_sum_slot<D, VEC>(c0 + e)];
    r.qn[e] = s_q[1][q_sum_slot<D, VEC>(c0 + e)];
  }
  return r;
}

template <int D, int G, int VEC>
__device__ __forceinline__ QSums<VEC> q_sums_shared(const float (&qc)[G], double (&s_q)[2][D],
                                                    int c0) {
  if (threadIdx.x < D) {
    double p = 0.0, n = 0.0;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const double x = (double)qc[g];
      p += x >= 0.0 ? x : 0.0;
      n += x >= 0.0 ? 0.0 : x;
    }
    s_q[0][q_sum_slot<D, VEC>(threadIdx.x)] = p;
    s_q[1][q_sum_slot<D, VEC>(threadIdx.x)] = n;
  }
  __syncthreads();
  return q_sums_read<D, VEC>(s_q, c0);
}

// Score of one page from its lo / hi slices, by the LPR lanes that hold the page (every lane
// returns the group's sum): the channel terms qp*hi + qn*lo (each product exact inside the fp64
// fma), folded over the LPR lanes.
template <int VEC, int LPR>
__device__ __forceinline__ double page_score(const QSums<VEC>& qs, const float* lo,
                                             const float* hi) {
  double acc = 0.0;
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    acc = fma(qs.qp[e], (double)hi[e], acc);
    acc = fma(qs.qn[e], (double)lo[e], acc);
  }
  return seg_sum_f64<LPR>(acc);
}

// Scores of chunk `chunk` (WAVES * U * 64 / LPR consecutive pages) of list (sequence b, KV head
// j), by one block of WAVES waves: LPR lanes read a page's lo and hi rows as 16-byte slices
// (sequence-major summaries: one contiguous run per wave and unroll step), take qp*hi + qn*lo per
// channel with the block's channel sums of the query (QSums) in fp64 fmas, and fold the LPR
// lanes; one fp64 -> fp32 rounding per score. Each
// lane group scores U pages (U > 1 for wide tables: fewer blocks, more loads in flight per lane).
// With the tail refresh on, the block holding the sequence's last page first rebuilds that page's
// summary from the key pool -- every wave folds a share of the tile's rows, the waves meet in LDS
// -- and the wave that scores the page writes the summary and scores it from the fresh values.
template <typename T, int D, int G, int WAVES, int U = 1, bool FP8 = false>
__device__ __forceinline__ void score_block(const SelectArgs& a, int j, int b, int chunk) {
  using M = row_map<T, D>;
  constexpr int VEC = M::VEC, LPR = M::LPR;
  constexpr int PPW = 64 / LPR;          // pages per wave and unroll step
  constexpr int PPB = WAVES * PPW * U;   // pages per block
  constexpr int NPT = (PPB + 63) / 64;   // page-id loads per lane (the block's pages)

  const int list = b * a.Hkv + j;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int P = a.P;
  const int pb0 = chunk * PPB;            // first page of this block
  const int wn0 = pb0 + w * PPW * U;      // first page of this wave
  const int Hq = a.Hkv * G;
  const T* q = (const T*)a.q;
  const int c0 = (lane % LPR) * VEC;
  const int rgl = lane / LPR;  // the lane's row group: page wn0 + u * PPW + rgl at step u

  // ---- loads first (unconditional, clamped addresses), all in one round: the block's page ids
  // (used only for the tail refresh), query channels, summary rows (sequence-major, so no page-table hop)
  // and the sequence length ----
  // the page ids first: the block that refreshes the tail page waits for them alone (loads
  // complete in issue order) and sends its key-tile loads while the summary rows are in flight
  // (entries past the sequence may hold anything and are clamped into the pool, never used)
  int pt_raw[NPT];
#pragma unroll
  for (int k = 0; k < NPT; ++k)  // indices from the row width only: no wait for seq_lens
    pt_raw[k] = a.page_table[(size_t)b * a.maxp + min(pb0 + k * 64 + lane, a.maxn - 1)];
  // the query, one channel per thread, for the block's channel sums
  static_assert(WAVES * 64 >= D, "one thread per channel");
  float qc[G];
  q_channel_load<T, D, G>(q + ((size_t)b * Hq + j * G) * D, qc);
  uint4 lo_raw[U], hi_raw[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int nc = min(wn0 + u * PPW + rgl, a.maxn - 1);
    const T* srow = (const T*)a.summ + ((size_t)list * a.maxp + nc) * 2 * D + c0;
    lo_raw[u] = load16_nt(srow);
    hi_raw[u] = load16_nt(srow + D);
  }
  __builtin_amdgcn_sched_barrier(0);
  const int L = a.seq_lens[b];
  const int N = L > 0 ? min((L + P - 1) / P, a.maxn) : 0;  // never past the live bound

  // ---- the decode-time refresh: the sequence's last page, the block and the wave holding it ----
  const int nt = N - 1;
  const int to = nt - pb0;  // the tail page's place in the block
  const bool btail = a.refresh_tail && N > 0 && to >= 0 && to < PPB;  // block-uniform
  const bool tail = btail && nt >= wn0 && nt < wn0 + PPW * U;         // wave-uniform

  if constexpr (U == 1) {
    const int t_off = nt - wn0;
    const int ut = tail ? t_off / PPW : -1, rg = t_off % PPW;  // its unroll step and row group
    float flo[VEC], fhi[VEC];
    if (btail) {
      int pt = 0;
#pragma unroll
      for (int k = 0; k < NPT; ++k) {  // scalar selects (a uniform index into pt_raw would spill it)
        const int x = __builtin_amdgcn_readlane(pt_raw[k], to & 63);
        pt = k == (to >> 6) ? x : pt;
      }
      pt = min(max(pt, 0), a.Npp - 1);
      const size_t t = (size_t)pt * a.Hkv + j;
      float ksc = 1.0f;
      if constexpr (FP8) ksc = a.k_scale[t];  // in flight with the tile
      float plo[VEC], phi[VEC];
      if constexpr (FP8)
        tile_rows_minmax<T, D, WAVES, true>((const uint8_t*)a.k_pool + t * P * D, L - nt * P,
                                            a.page_fill, P, lane, w, pt, 0, a.rope, plo, phi);
      else
        tile_rows_minmax<T, D, WAVES, false>((const T*)a.k_pool + t * P * D, L - nt * P,
                                             a.page_fill, P, lane, w, pt,
                                             rope_row_index(a.rope, b, nt, pt), a.rope, plo, phi);
      const int off = fold_lanes_scatter<LPR, VEC>(plo, phi);
      __shared__ __align__(16) float s_fold[WAVES][2][D];  // each wave's extremes of the tile
#pragma unroll
      for (int i = 0; i < scatter_kept<LPR, VEC>(); ++i) {
        s_fold[w][0][c0 + off + i] = plo[i];
        s_fold[w][1][c0 + off + i] = phi[i];
      }
      __syncthreads();
      if (tail) {
#pragma unroll
        for (int e = 0; e < VEC; e += 4) {
          const float4 l0 = *(const float4*)&s_fold[0][0][c0 + e];
          const float4 h0 = *(const float4*)&s_fold[0][1][c0 + e];
          flo[e] = l0.x, flo[e + 1] = l0.y, flo[e + 2] = l0.z, flo[e + 3] = l0.w;
          fhi[e] = h0.x, fhi[e + 1] = h0.y, fhi[e + 2] = h0.z, fhi[e + 3] = h0.w;
        }
#pragma unroll
        for (int v = 1; v < WAVES; ++v) {
#pragma unroll
          for (int e = 0; e < VEC; e += 4) {
            const float4 l = *(const float4*)&s_fold[v][0][c0 + e];
            const float4 h = *(const float4*)&s_fold[v][1][c0 + e];
            flo[e] = tmin(flo[e], l.x), flo[e + 1] = tmin(flo[e + 1], l.y);
            flo[e + 2] = tmin(flo[e + 2], l.z), flo[e + 3] = tmin(flo[e + 3], l.w);
            fhi[e] = tmax(fhi[e], h.x), fhi[e + 1] = tmax(fhi[e + 1], h.y);
            fhi[e + 2] = tmax(fhi[e + 2], h.z), fhi[e + 3] = tmax(fhi[e + 3], h.w);
          }
        }
        if constexpr (FP8) fp8_scale_outward<VEC>(ksc, flo, fhi);
        if (lane < LPR) {
          T* out = (T*)a.summ + ((size_t)list * a.maxp + nt) * 2 * D;
          store16(out + c0, pack<T>(flo));
          store16(out + D + c0, pack<T>(fhi));
        }
      }
    }

    // ---- scores of this wave's pages ----
    __shared__ double s_q[2][D];  // the block's channel sums
    const QSums<VEC> qs = q_sums_shared<D, G, VEC>(qc, s_q, c0);
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
      const double acc = page_score<VEC, LPR>(qs, lo, hi);
      const int n = wn0 + u * PPW + rgl;
      if (n < N && (lane % LPR) == 0) a.scores[(size_t)list * a.maxp + n] = (float)acc;
    }
  } else {
    // ---- scores of this wave's pages from the stored summary rows (the refreshed tail page's is
    // written from its fresh summary) ----
    __shared__ double s_q[2][D];  // the block's channel sums
    auto score_pages = [&](const QSums<VEC>& qs, int skip) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float lo[VEC], hi[VEC];
        unpack<T>(lo_raw[u], lo);
        unpack<T>(hi_raw[u], hi);
        const double acc = page_score<VEC, LPR>(qs, lo, hi);
        const int n = wn0 + u * PPW + rgl;
        if (n < N && n != skip && (lane % LPR) == 0) a.scores[(size_t)list * a.maxp + n] = (float)acc;
      }
    };
    if (!btail) {
      score_pages(q_sums_shared<D, G, VEC>(qc, s_q, c0), -1);
      return;
    }

    // ---- the block holding the tail page: its key tile's loads go out first (the page id is in
    // the lanes already); every wave folds its share of the tile's rows, the shares meet in LDS, and
    // the wave that scores the tail page combines them, scores the page and writes its summary.
    // The waves score their other pages while the tile is in flight ----
    int pt = 0;
#pragma unroll
    for (int k = 0; k < NPT; ++k) {  // scalar selects (a uniform index into pt_raw would spill it)
      const int x = __builtin_amdgcn_readlane(pt_raw[k], to & 63);
      pt = k == (to >> 6) ? x : pt;
    }
    pt = min(max(pt, 0), a.Npp - 1);
    const size_t t = (size_t)pt * a.Hkv + j;
    float ksc = 1.0f;
    if constexpr (FP8) ksc = a.k_scale[t];  // in flight with the tile
    TileMinMax<T, D, WAVES, FP8> tm;
    if constexpr (FP8)
      tm.start((const uint8_t*)a.k_pool + t * P * D, L - nt * P, a.page_fill, P, lane, w, pt, 0,
               a.rope);
    else
      tm.start((const T*)a.k_pool + t * P * D, L - nt * P, a.page_fill, P, lane, w, pt,
               rope_row_index(a.rope, b, nt, pt), a.rope);
    {
      // the scoring must stay behind the tile loads: these registers, renamed here, keep the
      // compiler from hoisting its (identical) start above the branch
#pragma unroll
      for (int g = 0; g < G; ++g) asm volatile("" : "+v"(qc[g]));
#pragma unroll
      for (int u = 0; u < U; ++u) {
        asm volatile("" : "+v"(lo_raw[u].x), "+v"(lo_raw[u].y), "+v"(lo_raw[u].z), "+v"(lo_raw[u].w));
        asm volatile("" : "+v"(hi_raw[u].x), "+v"(hi_raw[u].y), "+v"(hi_raw[u].z), "+v"(hi_raw[u].w));
      }
      score_pages(q_sums_shared<D, G, VEC>(qc, s_q, c0), nt);
    }
    float plo[VEC], phi[VEC];
    tm.finish(a.rope, plo, phi);
    const int off = fold_lanes_scatter<LPR, VEC>(plo, phi);
    __shared__ __align__(16) float s_fold[WAVES][2][D];  // each wave's extremes of the tile
#pragma unroll
    for (int i = 0; i < scatter_kept<LPR, VEC>(); ++i) {
      s_fold[w][0][c0 + off + i] = plo[i];
      s_fold[w][1][c0 + off + i] = phi[i];
    }
    __syncthreads();
    if (!tail) return;
    float flo[VEC], fhi[VEC];
#pragma unroll
    for (int e = 0; e < VEC; e += 4) {
      const float4 l0 = *(const float4*)&s_fold[0][0][c0 + e];
      const float4 h0 = *(const float4*)&s_fold[0][1][c0 + e];
      flo[e] = l0.x, flo[e + 1] = l0.y, flo[e + 2] = l0.z, flo[e + 3] = l0.w;
      fhi[e] = h0.x, fhi[e + 1] = h0.y, fhi[e + 2] = h0.z, fhi[e + 3] = h0.w;
    }
#pragma unroll
    for (int v = 1; v < WAVES; ++v) {
#pragma unroll
      for (int e = 0; e < VEC; e += 4) {
        const float4 l = *(const float4*)&s_fold[v][0][c0 + e];
        const float4 h = *(const float4*)&s_fold[v][1][c0 + e];
        flo[e] = tmin(flo[e], l.x), flo[e + 1] = tmin(flo[e + 1], l.y);
        flo[e + 2] = tmin(flo[e + 2], l.z), flo[e + 3] = tmin(flo[e + 3], l.w);
        fhi[e] = tmax(fhi[e], h.x), fhi[e + 1] = tmax(fhi[e + 1], h.y);
        fhi[e + 2] = tmax(fhi[e + 2], h.z), fhi[e + 3] = tmax(fhi[e + 3], h.w);
      }
    }
    if constexpr (FP8) fp8_scale_outward<VEC>(ksc, flo, fhi);
    const double acc = page_score<VEC, LPR>(q_sums_read<D, VEC>(s_q, c0), flo, fhi);  // every row group: the same page
    if (lane == 0) a.scores[(size_t)list * a.maxp + nt] = (float)acc;
    if (lane < LPR) {
      T* out = (T*)a.summ + ((size_t)list * a.maxp + nt) * 2 * D;
      store16(out + c0, pack<T>(flo));
      store16(out + D + c0, pack<T>(fhi));
    }
  }
}

// Unroll (pages per lane group) of the score kernel for a live page bound and a list count: long
// lists take fewer, fuller blocks. Measured with non-temporal summary reads:
// - at 1024 pages, U = 1 / 2 / 4 gave the 32K step in 14.15 / 14.54 / 15.21 us;
// - at 4096 pages and 8 lists, U = 2 / 4 gave the 128K selection call in 12.85 / 13.13 us;
// - at 128 lists of 4096 pages, U = 2 / 4 gave it in 68.0 / 55.3 us.
inline int score_unroll(int maxn, int nlists) {
  if (maxn <= 1024) return 1;
  if (maxn <= 2048 || (maxn <= 8192 && nlists < 64)) return 2;
  return 4;
}

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
