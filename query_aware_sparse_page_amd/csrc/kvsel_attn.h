// Sparse paged decode attention on the matrix cores: the per-block bodies shared by the split
// launch (attention.hip), the fused selection + attention launch (select_attend.hip) and the
// speculative step's co-scheduled launch (speculative.hip). Split-K over the selected pages, then
// a log-sum-exp merge of the splits in a second launch (attention.hip).
//
// Work unit: a "tile" of TT token slots (TT = 32 for bf16, 16 for fp32) taken in order from the
// concatenated selected pages of one list (= sequence, KV head). Grid: one block per
// (KV head, sequence, split) in a 3-D grid, KV head varying fastest, so that all splits of a list
// are placed on one XCD by the round-robin block placement when the number of lists is a multiple
// of 8, and no block index needs an integer division. A block has WAVES
// waves; each wave owns TPW consecutive tiles, issues every K and V load of its tiles first,
// then runs the contractions on MFMA with the GQA group of query heads as the M dimension
// (rows >= G are zero and ignored):
//
//  bf16 (v_mfma_f32_16x16x32_bf16; lane l: r16 = l % 16, q4 = l / 16):
//   S^T = K q^T per 16-token half h: A = K rows (16 tokens x 32 channels), B = q^T (32 channels x
//   16 heads). Row r of half h is token 8*(r/4) + 4h + r%4 of the tile, so after both halves
//   lane l holds the scores of head r16 for the 8 consecutive tokens 8*q4 .. 8*q4+7 -- exactly
//   the A operand of O = P V (16 heads x 32 tokens), with no data movement between lanes.
//   B = V (32 tokens x 16 channels) wants 8 consecutive tokens of one channel per lane: V pages
//   are stored channel-major ([D][P]), so that is one 16-byte load.
//  fp32 (v_mfma_f32_16x16x4f32): the same shape with 4-deep steps; step s of q K^T takes channel
//   (D/4)*q4 + s (a lane's 16-byte K loads cover its channels), step s of P V takes token
//   4*q4 + s (a lane's 16-byte V load covers its tokens).
//
// Softmax: per wave a two-pass max / exp over its tiles (the max needs 2 cross-lane steps),
// two row sums accumulated per lane -- l of the probabilities as they enter P V (bf16-rounded
// in the bf16 body, so the weights applied to V sum to one exactly) and lu of the unrounded fp32
// probabilities, which gives lse -- and O accumulated in the MFMA accumulators; the waves of a
// block merge through LDS. One split: the block writes out / lse directly. Otherwise it writes
// its (acc[G][D], m, l, lu) partial and attn_merge_kernel (one block per list) combines the
// partials in split order: M = max m_s, out = sum_s e^(m_s - M) acc_s / sum_s e^(m_s - M) l_s,
// lse = M + ln sum_s e^(m_s - M) lu_s.
// Invalid token slots (past a sequence's end, or past the list's count) load as zeros and get
// probability 0, so poisoned padding never reaches the accumulators.
#pragma once

#include <math.h>

#include "kvsel_device.h"
#include "kvsel_fp8.h"
#include "kvsel_internal.h"
#include "kvsel_topk.h"

namespace kvsel {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int ATT_MAX_SPLITS = 256;

struct AttnArgs {
  const void* k_pool;
  const void* v_pool;   // channel-major pages: [Npp][Hkv][D][P]
  const int32_t* page_table;
  const int32_t* seq_lens;
  const void* q;
  const int32_t* sel_idx;
  const int32_t* sel_cnt;
  int Hkv, P, log2P, maxp, Npp, k, pps, nsplit, nlists;
  int maxn;  // live pages at most (<= maxp, the row stride)
  float scale;
  const float* k_scale;  // fp8 pools: [Npp][Hkv] tile scales of K and V (else null)
  const float* v_scale;
  const int32_t* page_fill;  // [Npp] valid slots per physical page, or null (every page full)
  RopeArgs rope;
  float* part_acc;   // [nlists][nsplit][G][D]
  float4* part_ml;   // [nlists][nsplit][G]: (m, l, lu, unused)
  void* out;
  float* lse;
  // fused selection only: the scores, and the selection outputs written by split 0
  const float* scores;  // [nlists][maxp]
  int32_t* sel_out;     // [nlists][k]
  int32_t* cnt_out;     // [nlists]
  // speculative step only (fused selection): reuse.q_prev != nullptr makes every block read its
  // list's decision from reuse.corrected (written by an earlier launch); see select_tiles
  ReuseArgs reuse;
};

constexpr int ATT_MAX_PPS = 16;  // pages per split of the fused-selection launches

// Wave-uniform page lookup of the NPT pages a tile of TT token slots touches (NPT = 2 when a
// 32-slot tile spans two 16-slot pages). The addresses follow the selection id and page-table
// entry as read (an id out of range is clamped to a valid entry), and the list count only
// decides validity, so the dependent chain is id -> page table -> K / V with every id load in one
// round and every page-table load in the next.
template <int P, int TT, int TPW>
struct TilePages {
  static constexpr int NPT = TT > P ? TT / P : 1;
  static_assert(NPT <= 2, "a tile spans at most two pages");
  int page[TPW][NPT];   // physical page to address (always a valid page)
  int valid[TPW][NPT];  // valid slots of that page; 0 when the slot range is not in the list
  int lpage[TPW][NPT];  // its logical page in the sequence (the per-sequence rotary rows)
  // Entry u (lane-dependent, 0 or 1) of tile t, by arithmetic: a register array indexed by a
  // per-lane value (which a select of two entries can be folded into) lands in private memory.
  __device__ __forceinline__ int page_of(int t, int u) const {
    return NPT == 1 ? page[t][0] : page[t][0] + u * (page[t][NPT - 1] - page[t][0]);
  }
  __device__ __forceinline__ int lpage_of(int t, int u) const {
    return NPT == 1 ? lpage[t][0] : lpage[t][0] + u * (lpage[t][NPT - 1] - lpage[t][0]);
  }
  __device__ __forceinline__ int valid_of(int t, int u) const {
    return NPT == 1 ? valid[t][0] : valid[t][0] + u * (valid[t][NPT - 1] - valid[t][0]);
  }
};

template <int P, int TT, int TPW>
__device__ __forceinline__ void lookup_tiles(const AttnArgs& a, int list, int b, int split,
                                             int first_tile, TilePages<P, TT, TPW>& tp) {
  constexpr int NPT = TilePages<P, TT, TPW>::NPT;
  // the ids, the list count and the length are issued unconditionally from clamped indices and
  // held in front by a scheduling barrier, so they share one memory round trip (left to itself
  // the compiler issued the length after waiting for the ids)
  int n_raw[TPW][NPT];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int u = 0; u < NPT; ++u) {
      const int sp = split * a.pps + ((first_tile + t) * TT) / P + u;
      n_raw[t][u] = __builtin_amdgcn_readfirstlane(a.sel_idx[(size_t)list * a.k + min(sp, a.k - 1)]);
    }
  const int cnt_raw = __builtin_amdgcn_readfirstlane(a.sel_cnt[list]);
  const int L = __builtin_amdgcn_readfirstlane(a.seq_lens[b]);
  __builtin_amdgcn_sched_barrier(0);
  const int cnt = min(cnt_raw, a.k);
  int n[TPW][NPT];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int u = 0; u < NPT; ++u) {
      const int sp = split * a.pps + ((first_tile + t) * TT) / P + u;
      n[t][u] = sp < a.k ? n_raw[t][u] : -1;
    }
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int u = 0; u < NPT; ++u) {
      const int nn = n[t][u];
      const bool in_range = nn >= 0 && nn < a.maxp;
      // an entry outside the list may hold anything: clamp it into the pool before addressing
      const int pg = __builtin_amdgcn_readfirstlane(a.page_table[(size_t)b * a.maxp + (in_range ? nn : 0)]);
      tp.page[t][u] = min(max(pg, 0), a.Npp - 1);
      tp.lpage[t][u] = in_range ? nn : 0;
      const int sp = split * a.pps + ((first_tile + t) * TT) / P + u;
      tp.valid[t][u] = (in_range && sp < cnt) ? min(P, L - nn * P) : 0;
    }
}

// Fused selection (kvsel_select_attend): every block of a list re-derives the list's top-k from
// the page scores with the block-wide radix select and keeps the pages of its own split. The
// scores and the page-table row are loaded together, so the K / V loads follow one memory round
// trip and the select, instead of the selection ids -> page table -> K / V chain. The block of
// split 0 also writes the selection outputs.
// In the speculative step (a.reuse.q_prev != nullptr), corr is the list's reuse decision. A list
// kept on the previous step's pages (corr == 0) already has its partials from those pages: its
// blocks other than split 0 return right after the loads, and its split-0 block writes the
// selection outputs plus used = the previous list, then returns. A corrected list also gets
// used = its fresh selection. Returns whether the block goes on to attend.
template <int NT>
struct SplitSelectSmem {
  RadixSmem<NT> r;
  int page[ATT_MAX_PPS];   // physical page at each of the split's positions
  int valid[ATT_MAX_PPS];  // its valid slots (0: nothing selected at that position)
  int lpage[ATT_MAX_PPS];  // its logical page
};

template <int P, int TT, int TPW, int NT, int C>
__device__ __forceinline__ bool select_tiles(const AttnArgs& a, int list, int b, int split,
                                             int first_tile, int corr, TilePages<P, TT, TPW>& tp,
                                             SplitSelectSmem<NT>& ss) {
  constexpr int NPT = TilePages<P, TT, TPW>::NPT;
  const int tid = threadIdx.x;
  const float* sc = a.scores + (size_t)list * a.maxp;
  const int32_t* row = a.page_table + (size_t)b * a.maxp;
  float v[C];
  int pt[C];
#pragma unroll
  for (int u = 0; u < C; ++u) {  // indices from the live bound only: no wait for seq_lens
    const int i = min(tid * C + u, a.maxn - 1);
    v[u] = sc[i];
    pt[u] = row[i];
  }
  const int L = a.seq_lens[b];
  if (!corr && split != 0) return false;  // block-uniform
  const int N = L > 0 ? min((L + P - 1) / P, a.maxn) : 0;
  const int first = split * a.pps;
  // positions of this split past the selection's length are never filled: clear those (the
  // others are written exactly once by the select, so no barrier is needed before it)
  if (tid < a.pps && first + tid >= min(N, a.k)) {
    ss.page[tid] = 0;
    ss.valid[tid] = 0;
    ss.lpage[tid] = 0;
  }
  uint32_t key[C];
#pragma unroll
  for (int u = 0; u < C; ++u) key[u] = score_key(v[u]);
  const bool writer = split == 0 && a.sel_out != nullptr;
  const bool spec = a.reuse.q_prev != nullptr;
  int32_t* out = a.sel_out + (size_t)list * a.k;
  int32_t* used = (writer && spec && corr) ? a.reuse.used_idx + (size_t)list * a.k : nullptr;
  block_topk_regs<NT, C>(key, N, a.k, ss.r, [&](int pos, int i, int u) {
    if (writer) {
      out[pos] = i;
      if (used) used[pos] = i;
    }
    const int sp = pos - first;
    if (sp >= 0 && sp < a.pps) {
      ss.page[sp] = min(max(pt[u], 0), a.Npp - 1);  // any table value stays inside the pool
      ss.valid[sp] = min(P, L - i * P);
      ss.lpage[sp] = i;
    }
  });
  if (writer) {
    const int cnt = min(N, a.k);
    for (int i = cnt + tid; i < a.k; i += NT) {
      out[i] = -1;
      if (used) used[i] = -1;
    }
    if (tid == 0) a.cnt_out[list] = cnt;
    if (spec && corr && tid == 0) a.reuse.used_cnt[list] = cnt;
    if (spec && !corr) {  // kept on the previous step's pages
      for (int i = tid; i < a.k; i += NT)
        a.reuse.used_idx[(size_t)list * a.k + i] = a.reuse.prev_idx[(size_t)list * a.k + i];
      if (tid == 0) a.reuse.used_cnt[list] = a.reuse.prev_cnt[list];
    }
  }
  if (!corr) return false;  // block-uniform: this split's partial is already in place
  __syncthreads();
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int u = 0; u < NPT; ++u) {
      const int sp = ((first_tile + t) * TT) / P + u;
      tp.page[t][u] = __builtin_amdgcn_readfirstlane(ss.page[sp]);
      tp.valid[t][u] = __builtin_amdgcn_readfirstlane(ss.valid[sp]);
      tp.lpage[t][u] = __builtin_amdgcn_readfirstlane(ss.lpage[sp]);
    }
  return true;
}

// Rotate-half rotation of one channel pair held by the same lane (bits identical to
// rope_rotate_slice).
template <typename T>
__device__ __forceinline__ void rope_pair(float& x1, float& x2, float c, float s) {
  const float y1 = rot_sub(rot_mul(x1, c), rot_mul(x2, s));
  const float y2 = rot_add(rot_mul(x2, c), rot_mul(x1, s));
  x1 = round_to_elem<T>(y1);
  x2 = round_to_elem<T>(y2);
}

// The rotation of rope_pair without its rounding (the gather packs the results once, below).
__device__ __forceinline__ void rope_pair_f32(float& x1, float& x2, float c, float s) {
  const float y1 = rot_sub(rot_mul(x1, c), rot_mul(x2, s));
  const float y2 = rot_add(rot_mul(x2, c), rot_mul(x1, s));
  x1 = y1;
  x2 = y2;
}

// 8 fp32 values to 8 bf16 by gfx950's packed conversion (round to nearest even: for every finite
// value the bits of round_to_elem<bf16_t>, one instruction per pair instead of the integer
// sequence).
__device__ __forceinline__ uint4 pack_bf16x8_rne(const float* f) {
  typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2_v v = {(__bf16)f[2 * i], (__bf16)f[2 * i + 1]};
    __builtin_memcpy(&w[i], &v, 4);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) {
  bf16x8_t r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

__device__ __forceinline__ uint4 pack_bf16x8(const float* f) { return pack<bf16_t>(f); }

// Zero the bf16 elements e of v whose bit e of `keep` is clear (invalid token slots).
__device__ __forceinline__ uint4 mask_bf16x8(const uint4& v, int keep) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] &= ((keep >> (2 * i)) & 1 ? 0x0000ffffu : 0u) | ((keep >> (2 * i + 1)) & 1 ? 0xffff0000u : 0u);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Zero the fp32 elements e of v whose bit e of `keep` is clear.
__device__ __forceinline__ uint4 mask_f32x4(const uint4& v, int keep) {
  return make_uint4((keep & 1) ? v.x : 0u, (keep & 2) ? v.y : 0u, (keep & 4) ? v.z : 0u,
                    (keep & 8) ? v.w : 0u);
}

constexpr int ATT_MAX_G = 8;

// Block-level merge of the waves' (m, l, lu, O) and the write of the block's result. The weight
// e^(m_v - M) of each (wave, head) is computed once, by G threads, before the channels combine.
// A wave without a valid token has m = -inf and O = 0, and gets weight 0.
template <typename T, int D, int WAVES>
__device__ __forceinline__ void finish_block(const AttnArgs& a, int G, int list, int split, int b,
                                             int j, float (*s_m)[ATT_MAX_G],
                                             float (*s_l)[ATT_MAX_G], float (*s_lu)[ATT_MAX_G],
                                             float (*s_o)[ATT_MAX_G][D]) {
  const float NEG_INF = __int_as_float(0xff800000);
  const int Hq = a.Hkv * G;
  __shared__ float s_w[WAVES][ATT_MAX_G], s_blk[3][ATT_MAX_G];  // weights; the block's M, l, lu
  __syncthreads();
  if (threadIdx.x < G) {
    const int g = threadIdx.x;
    float Mx = s_m[0][g];
#pragma unroll
    for (int v = 1; v < WAVES; ++v) Mx = fmaxf(Mx, s_m[v][g]);
    float Ls = 0.0f, Lu = 0.0f;
#pragma unroll
    for (int v = 0; v < WAVES; ++v) {
      const float f = (Mx != NEG_INF && s_m[v][g] != NEG_INF) ? __expf(s_m[v][g] - Mx) : 0.0f;
      s_w[v][g] = f;
      Ls = fmaf(s_l[v][g], f, Ls);
      Lu = fmaf(s_lu[v][g], f, Lu);
    }
    s_blk[0][g] = Mx;
    s_blk[1][g] = Ls;
    s_blk[2][g] = Lu;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += WAVES * 64) {
    const int g = idx / D, d = idx % D;
    float A = 0.0f;
#pragma unroll
    for (int v = 0; v < WAVES; ++v) A = fmaf(s_o[v][g][d], s_w[v][g], A);
    const float Mx = s_blk[0][g], Ls = s_blk[1][g], Lu = s_blk[2][g];
    if (a.nsplit == 1) {
      const size_t o = ((size_t)b * Hq + j * G + g) * D + d;
      store_elem<T>((T*)a.out, o, Mx == NEG_INF ? 0.0f : A / Ls);
      if (d == 0 && a.lse)
        a.lse[(size_t)b * Hq + j * G + g] = Mx == NEG_INF ? NEG_INF : Mx + logf(Lu);
    } else {
      const size_t ps = ((size_t)list * a.nsplit + split) * G + g;
      a.part_acc[ps * D + d] = A;
      if (d == 0) a.part_ml[ps] = make_float4(Mx, Ls, Lu, 0.0f);
    }
  }
}

// ------------------------------------------------------------------------------------------
// bf16
// ------------------------------------------------------------------------------------------
// SEL_C > 0: fused selection with SEL_C score keys per thread (select_tiles).
// FP8: the pools hold E4M3 codes with per-tile scales. A lane's K and V loads are then 8 bytes
// (8 codes) where bf16 loads 16, decoded to bf16 exactly after every load has been issued, so the
// MFMA layouts are unchanged. A lane's 8 tokens of a tile lie in one page, so one (k_scale,
// v_scale) pair per lane and tile: the logits take scale * k_scale, and each probability enters
// P V as bf16(p * v_scale) while l adds bf16(p).
// FILL: the pages may end early (page_fill, composed sequences); a separate instantiation, so
// the common case carries none of its registers.
template <int D, int P, int WAVES, int TPW, bool ROPE, int SEL_C = 0, bool FP8 = false,
          bool FILL = false>
__device__ __forceinline__ void attn_bf16_block(const AttnArgs& a, int G, int j, int b, int split) {
  static_assert(!(FP8 && ROPE), "fp8 pools take no rotary gather");
  constexpr int TT = 32;       // tokens per tile
  constexpr int CB = D / 32;   // 32-channel blocks of q K^T
  constexpr int VB = D / 16;   // 16-channel blocks of P V
  using TP = TilePages<P, TT, TPW>;
  const float NEG_INF = __int_as_float(0xff800000);
  const int list = b * a.Hkv + j;
  // the list's speculative-reuse decision, loaded first (fused selection only)
  int corr = 1;
  if constexpr (SEL_C > 0) {
    if (a.reuse.q_prev) corr = __builtin_amdgcn_readfirstlane((int)a.reuse.corrected[list]);
  }
  (void)corr;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, q4 = lane >> 4;
  const int Hq = a.Hkv * G;
  const bf16_t* kp = (const bf16_t*)a.k_pool;
  const bf16_t* vp = (const bf16_t*)a.v_pool;

  // q^T operand (independent of the selection): q[head r16][32 cb + 8 q4 .. +8], zero rows >= G
  // (loads below are unconditional, from clamped valid addresses, and masked where used: a
  // conditional load makes the compiler wait for it before issuing the next one)
  uint4 qraw[CB];
  {
    const bf16_t* qrow = (const bf16_t*)a.q + ((size_t)b * Hq + j * G + min(r16, G - 1)) * D + 8 * q4;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) qraw[cb] = load16(qrow + 32 * cb);
  }

  TP tp;
  if constexpr (SEL_C > 0) {
    __shared__ SplitSelectSmem<WAVES * 64> ss;
    if (!select_tiles<P, TT, TPW, WAVES * 64, SEL_C>(a, list, b, split, w * TPW, corr, tp, ss))
      return;
  } else {
    lookup_tiles<P, TT, TPW>(a, list, b, split, w * TPW, tp);
  }

  // ---- every K / V load of this wave's tiles ----
  uint4 kraw[TPW][2][CB], vraw[TPW][VB];
  [[maybe_unused]] uint2 k8[TPW][2][CB], v8[TPW][VB];  // fp8 codes (FP8 only)
  [[maybe_unused]] float ksc[TPW], vsc[TPW];  // the lane's page's tile scales (FP8 only)
  int vmask[TPW];  // bit e set: token 8*q4 + e of the tile is valid
  int krow[TPW][2];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int x = 8 * (r16 / 4) + 4 * h + (r16 % 4);  // token of row r16 in half h
      const int u = x / P, slot = x % P;
      const int pg = tp.page_of(t, u);
      // an invalid token's row of S^T is masked to -inf below (rows of an MFMA are
      // independent), so its K needs no zeroing
      const size_t krow_off = (((size_t)pg * a.Hkv + j) * P + slot) * D + 8 * q4;
      if constexpr (FP8) {
        const uint8_t* row = (const uint8_t*)a.k_pool + krow_off;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) k8[t][h][cb] = load8_nt(row + 32 * cb);
      } else {
        const bf16_t* row = kp + krow_off;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) kraw[t][h][cb] = load16_nt(row + 32 * cb);
      }
      if (ROPE) {
        const int pr = a.rope.page_row[rope_row_index(a.rope, b, tp.lpage_of(t, u), pg)];
        krow[t][h] = pr < 0 ? -1 : pr + a.rope.row_step * slot;
      }
    }
    const int xv = 8 * q4;  // first of the lane's 8 value tokens
    const int u = xv / P, slot = xv % P;
    const int pg = tp.page_of(t, u);
    int m = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) m |= (slot + e < tp.valid_of(t, u)) ? (1 << e) : 0;
    vmask[t] = m;
    const size_t vt_off = ((size_t)pg * a.Hkv + j) * D * P + slot + (size_t)r16 * P;
    if constexpr (FP8) {
      const uint8_t* vt = (const uint8_t*)a.v_pool + vt_off;
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) v8[t][vb] = load8_nt(vt + (size_t)(16 * vb) * P);
      ksc[t] = a.k_scale[(size_t)pg * a.Hkv + j];
      vsc[t] = a.v_scale[(size_t)pg * a.Hkv + j];
    } else {
      const bf16_t* vt = vp + vt_off;
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) vraw[t][vb] = load16_nt(vt + (size_t)(16 * vb) * P);
    }
  }
  // valid slots of the tiles' pages in a composed sequence (page_fill): scalar loads after the
  // K / V loads, applied to the masks
  [[maybe_unused]] int fillp[TPW][TP::NPT];
  if constexpr (FILL) {
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int u = 0; u < TP::NPT; ++u)
        fillp[t][u] = __builtin_amdgcn_readfirstlane(a.page_fill[tp.page[t][u]]);
  }
  __builtin_amdgcn_sched_barrier(0);  // keep every load above the first use
  if constexpr (FILL) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int xv = 8 * q4, u = xv / P, slot = xv % P;
      const int f = TP::NPT == 1 ? fillp[t][0]
                                 : fillp[t][0] + u * (fillp[t][TP::NPT - 1] - fillp[t][0]);
      int m = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) m |= (slot + e < f) ? (1 << e) : 0;
      vmask[t] &= m;
    }
  }
  if constexpr (FP8) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) kraw[t][h][cb] = fp8x8_to_bf16x8(k8[t][h][cb]);
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) vraw[t][vb] = fp8x8_to_bf16x8(v8[t][vb]);
    }
  }

  // ---- S^T = K q^T ----
  f32x4_t s[TPW][2];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (ROPE) {
        // rotate-half pairs (c, c + D/2) sit in blocks cb and cb + CB/2 of the same lane
        const int row = krow[t][h];
        if (row >= 0) {
#pragma unroll
          for (int cb = 0; cb < CB / 2; ++cb) {
            float x1[8], x2[8];
            unpack<bf16_t>(kraw[t][h][cb], x1);
            unpack<bf16_t>(kraw[t][h][cb + CB / 2], x2);
            const float* cr = a.rope.cos + (size_t)row * (D / 2) + 32 * cb + 8 * q4;
            const float* sr = a.rope.sin + (size_t)row * (D / 2) + 32 * cb + 8 * q4;  // row >= 0 here
            float cv[8], sv[8];
            unpack<float>(load16(cr), cv);
            unpack<float>(load16(cr + 4), cv + 4);
            unpack<float>(load16(sr), sv);
            unpack<float>(load16(sr + 4), sv + 4);
#pragma unroll
            for (int e = 0; e < 8; ++e) rope_pair_f32(x1[e], x2[e], cv[e], sv[e]);
            kraw[t][h][cb] = pack_bf16x8_rne(x1);
            kraw[t][h][cb + CB / 2] = pack_bf16x8_rne(x2);
          }
        }
      }
      f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kraw[t][h][cb]), as_bf16x8(qraw[cb]),
                                                      acc, 0, 0, 0);
      s[t][h] = acc;
    }
  }

  // ---- softmax over the wave's tokens (head r16; tokens 8*q4 + 4h + i of each tile) ----
  float z[TPW][8];
  float m = NEG_INF;
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const float sc = FP8 ? a.scale * ksc[t] : a.scale;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = s[t][e >> 2][e & 3] * sc;
      z[t][e] = ((vmask[t] >> e) & 1) && r16 < G ? v : NEG_INF;
      m = fmaxf(m, z[t][e]);
    }
  }
  m = fmaxf(m, xor16_f32(m));
  m = fmaxf(m, xor32_f32(m));
  float l = 0.0f, lu = 0.0f;
  f32x4_t o[VB];
#pragma unroll
  for (int vb = 0; vb < VB; ++vb) o[vb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    // P enters the MFMA as bf16: normalize by the sum of the rounded values, so the weights
    // applied to V sum to one exactly (fp8: l sums bf16(p), the MFMA takes bf16(p * v_scale));
    // lse takes the sum of the unrounded values
    float pf[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pf[e] = z[t][e] == NEG_INF ? 0.0f : __expf(z[t][e] - m);
      lu += pf[e];
    }
    uint4 pb;
    if constexpr (FP8) {
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = pf[e] * vsc[t];
      pb = pack_bf16x8_rne(pv);
    } else {
      pb = pack_bf16x8_rne(pf);
    }
    {
      const uint4 lb = FP8 ? pack_bf16x8_rne(pf) : pb;
      const uint32_t lw[4] = {lb.x, lb.y, lb.z, lb.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        l += __uint_as_float(lw[i] << 16);
        l += __uint_as_float(lw[i] & 0xffff0000u);
      }
    }
    const bf16x8_t pa = as_bf16x8(pb);
    const bool partial = vmask[t] != 0xff;  // zero invalid slots (0 * NaN poison is NaN)
#pragma unroll
    for (int vb = 0; vb < VB; ++vb) {
      const uint4 vv = partial ? mask_bf16x8(vraw[t][vb], vmask[t]) : vraw[t][vb];
      o[vb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, as_bf16x8(vv), o[vb], 0, 0, 0);
    }
  }
  l += xor16_f32(l);
  l += xor32_f32(l);
  lu += xor16_f32(lu);
  lu += xor32_f32(lu);

  // ---- merge the block's waves through LDS ----
  __shared__ float s_m[WAVES][ATT_MAX_G], s_l[WAVES][ATT_MAX_G], s_lu[WAVES][ATT_MAX_G];
  __shared__ float s_o[WAVES][ATT_MAX_G][D];
  if (q4 == 0 && r16 < G) {
    s_m[w][r16] = m;
    s_l[w][r16] = l;
    s_lu[w][r16] = lu;
  }
  if (4 * q4 < G) {  // lanes holding rows (heads) 4*q4 .. 4*q4+3
#pragma unroll
    for (int vb = 0; vb < VB; ++vb)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_o[w][4 * q4 + i][16 * vb + r16] = o[vb][i];
  }
  finish_block<bf16_t, D, WAVES>(a, G, list, split, b, j, s_m, s_l, s_lu, s_o);
}

// ------------------------------------------------------------------------------------------
// fp32
// ------------------------------------------------------------------------------------------
template <int D, int P, int WAVES, int TPW, bool ROPE, int SEL_C = 0, bool FILL = false>
__device__ __forceinline__ void attn_f32_block(const AttnArgs& a, int G, int j, int b, int split) {
  constexpr int TT = 16;       // tokens per tile
  constexpr int KC = D / 4;    // channels per lane in q K^T (4 lane groups)
  constexpr int KL = KC / 4;   // 16-byte loads per lane per token
  constexpr int VB = D / 16;   // 16-channel blocks of P V
  using TP = TilePages<P, TT, TPW>;
  const float NEG_INF = __int_as_float(0xff800000);
  const int list = b * a.Hkv + j;
  // the list's speculative-reuse decision, loaded first (fused selection only)
  int corr = 1;
  if constexpr (SEL_C > 0) {
    if (a.reuse.q_prev) corr = __builtin_amdgcn_readfirstlane((int)a.reuse.corrected[list]);
  }
  (void)corr;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, q4 = lane >> 4;
  const int Hq = a.Hkv * G;
  const float* kp = (const float*)a.k_pool;
  const float* vp = (const float*)a.v_pool;

  float qv[KC];
  {
    // unconditional loads from clamped addresses, masked where used (see the bf16 kernel)
    const float* qrow = (const float*)a.q + ((size_t)b * Hq + j * G + min(r16, G - 1)) * D + KC * q4;
#pragma unroll
    for (int u = 0; u < KL; ++u) unpack<float>(load16(qrow + 4 * u), qv + 4 * u);
    if (r16 >= G) {
#pragma unroll
      for (int c = 0; c < KC; ++c) qv[c] = 0.0f;
    }
  }
  TP tp;
  if constexpr (SEL_C > 0) {
    __shared__ SplitSelectSmem<WAVES * 64> ss;
    if (!select_tiles<P, TT, TPW, WAVES * 64, SEL_C>(a, list, b, split, w * TPW, corr, tp, ss))
      return;
  } else {
    lookup_tiles<P, TT, TPW>(a, list, b, split, w * TPW, tp);
  }

  uint4 kraw[TPW][KL], vraw[TPW][VB];
  int vmask[TPW];
  int krow[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int tile = w * TPW + t;
    const int base = (tile * TT) % P;  // first slot of the tile within its page
    const int pg = tp.page[t][0];
    const int slot = base + r16;
    const float* row = kp + (((size_t)pg * a.Hkv + j) * P + slot) * D + KC * q4;
#pragma unroll
    for (int u = 0; u < KL; ++u) kraw[t][u] = load16_nt(row + 4 * u);
    if (ROPE) {
      const int pr = a.rope.page_row[rope_row_index(a.rope, b, tp.lpage[t][0], pg)];
      krow[t] = pr < 0 ? -1 : pr + a.rope.row_step * slot;
    }
    const int vslot = base + 4 * q4;
    int mk = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) mk |= (vslot + e < tp.valid[t][0]) ? (1 << e) : 0;
    vmask[t] = mk;
    const float* vt = vp + ((size_t)pg * a.Hkv + j) * D * P + vslot + (size_t)r16 * P;
#pragma unroll
    for (int vb = 0; vb < VB; ++vb) vraw[t][vb] = load16_nt(vt + (size_t)(16 * vb) * P);
  }
  [[maybe_unused]] int fillp[TPW];  // composed sequences: see attn_bf16_block
  if constexpr (FILL) {
#pragma unroll
    for (int t = 0; t < TPW; ++t)
      fillp[t] = __builtin_amdgcn_readfirstlane(a.page_fill[tp.page[t][0]]);
  }
  __builtin_amdgcn_sched_barrier(0);  // keep every load above the first use
  if constexpr (FILL) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int vslot = (w * TPW + t) * TT % P + 4 * q4;
      int mk = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) mk |= (vslot + e < fillp[t]) ? (1 << e) : 0;
      vmask[t] &= mk;
    }
  }

  f32x4_t s[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    float kv[KC];
#pragma unroll
    for (int u = 0; u < KL; ++u) unpack<float>(kraw[t][u], kv + 4 * u);
    if (ROPE) {
      // rotate-half partner of channel c (lane group q4) is in lane group q4 ^ 2; every lane
      // group of token r16 computed the same table row
      const int row = krow[t];
      float pv[KC];
#pragma unroll
      for (int e = 0; e < KC; ++e) pv[e] = lane_xor_f32(kv[e], 32);
      if (row >= 0) {
        const bool first = q4 < 2;
        const int i0 = first ? KC * q4 : KC * q4 - D / 2;
        const float* cr = a.rope.cos + (size_t)row * (D / 2) + i0;
        const float* sr = a.rope.sin + (size_t)row * (D / 2) + i0;
#pragma unroll
        for (int e = 0; e < KC; ++e) {
          float x1 = first ? kv[e] : pv[e], x2 = first ? pv[e] : kv[e];
          rope_pair<float>(x1, x2, cr[e], sr[e]);
          kv[e] = first ? x1 : x2;
        }
      }
    }
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < KC; ++c) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[c], qv[c], acc, 0, 0, 0);
    s[t] = acc;
  }
  float z[TPW][4];
  float m = NEG_INF;
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = s[t][i] * a.scale;
      z[t][i] = ((vmask[t] >> i) & 1) && r16 < G ? v : NEG_INF;
      m = fmaxf(m, z[t][i]);
    }
  m = fmaxf(m, xor16_f32(m));
  m = fmaxf(m, xor32_f32(m));
  float l = 0.0f;
  f32x4_t o[VB];
#pragma unroll
  for (int vb = 0; vb < VB; ++vb) o[vb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = z[t][i] == NEG_INF ? 0.0f : __expf(z[t][i] - m);
      l += p[i];
    }
    const bool partial = vmask[t] != 0xf;
#pragma unroll
    for (int vb = 0; vb < VB; ++vb) {
      float vv[4];
      unpack<float>(partial ? mask_f32x4(vraw[t][vb], vmask[t]) : vraw[t][vb], vv);
#pragma unroll
      for (int st = 0; st < 4; ++st)
        o[vb] = __builtin_amdgcn_mfma_f32_16x16x4f32(p[st], vv[st], o[vb], 0, 0, 0);
    }
  }
  l += xor16_f32(l);
  l += xor32_f32(l);

  // the probabilities enter the fp32 MFMA unrounded: l is both sums
  __shared__ float s_m[WAVES][ATT_MAX_G], s_l[WAVES][ATT_MAX_G];
  __shared__ float s_o[WAVES][ATT_MAX_G][D];
  if (q4 == 0 && r16 < G) {
    s_m[w][r16] = m;
    s_l[w][r16] = l;
  }
  if (4 * q4 < G) {
#pragma unroll
    for (int vb = 0; vb < VB; ++vb)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_o[w][4 * q4 + i][16 * vb + r16] = o[vb][i];
  }
  finish_block<float, D, WAVES>(a, G, list, split, b, j, s_m, s_l, s_l, s_o);
}


// ------------------------------------------------------------------------------------------
// shared host-side pieces
// ------------------------------------------------------------------------------------------
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Default split of the fused-selection launches and their block shape, which depends only on
// the dtype and page size and equals the split launch's shape for the same split:
//   bf16, P 32: 4 waves x 1 tile   bf16, P 16: 2 waves x 1 tile
//   fp32, P 32: 4 waves x 2 tiles  fp32, P 16: 4 waves x 1 tile
constexpr int FUSED_PPS = 4;

template <typename T, int P>
struct FusedShape {  // T = fp8_t: the bf16 shape (fp8 pages are decoded into the bf16 body)
  static constexpr int WAVES = (sizeof(T) <= 2 && P == 16) ? 2 : 4;
  static constexpr int TPW = (sizeof(T) == 4 && P == 32) ? 2 : 1;
};

// Attention arguments of one call; the partials live at ws when there is more than one split.
AttnArgs attn_args(const LaunchKV& kv, const RopeArgs& rope, const void* q, const int32_t* sel_idx,
                   const int32_t* sel_cnt, int k, float scale, int pps, void* out, float* lse,
                   void* ws);

// The merge launch of a.nsplit > 1 splits (nothing to do for one split).
hipError_t launch_merge(const LaunchKV& kv, const AttnArgs& a, hipStream_t stream);

// Fused selection + attention launch (the split launch with the top-k re-derived per block),
// then the merge; requires select_attend_fused(kv, rope, a.k) and a.pps == FUSED_PPS.
hipError_t launch_fused_select(const LaunchKV& kv, const AttnArgs& a, bool rope,
                               hipStream_t stream);

}  // namespace kvsel
