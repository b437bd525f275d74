// Speculative decode step ([FreeKV] section 2.1: step t attends over the pages selected at step
// t-1 unless the group-mean query similarity falls below tau, in which case it waits for this
// step's selection). Three launches on one stream:
//
//  1. co-launch, grid (Hkv, B, chunks + 1 + splits), one block shape: the blocks with z < chunks
//     score page chunks (score_block), z == chunks evaluates each list's reuse decision
//     (group_cosine, first wave), and the rest run the attention splits over the previous step's
//     pages (attn_*_block over prev_idx / prev_cnt) -- the attention that does not depend on this
//     step's selection shares the launch, and the chip, with the scoring. Score blocks have the
//     lowest z, so they are dispatched first.
//  2. the fused selection + attention launch in speculative mode: every block reads its list's
//     decision; a list kept on its previous pages only has its selection outputs written (split
//     0) and keeps the partials of launch 1; a corrected list is attended over its fresh pages,
//     overwriting them.
//  3. the merge of every list.
//
// The outputs equal those of kvsel_score_topk with reuse followed by kvsel_sparse_decode_attn
// over the used pages, bit for bit: the scores, the decision and the top-k run the same code, and
// every partial comes from the same block body over the same pages. The co-launch needs the
// fused selection's conditions (register-resident select, the default split); otherwise the two
// calls run serially. On the first step (every list corrected) launch 1 has no attention blocks.
// The speculative overlap across two streams (events between them) was slower on this GPU than
// the serial calls; a shared launch needs no cross-queue synchronization.
#include "kvsel_attn.h"
#include "kvsel_score.h"

namespace kvsel {

// T: the query / summary type (bf16 for fp8 pools, FP8 set).
template <typename T, int D, int P, bool ROPE, int G, bool FP8, int WAVES = FusedShape<T, P>::WAVES>
__global__ __launch_bounds__(WAVES * 64) void spec_co_kernel(AttnArgs a, SelectArgs s) {
  using S = FusedShape<T, P>;
  const int j = blockIdx.x, b = blockIdx.y, z = blockIdx.z;  // grid (Hkv, B, chunks + 1 + splits)
  if (z < s.nchunks) {  // chunks in reverse order: the tail refresh's blocks are dispatched first
    score_block<T, D, G, S::WAVES, 1, FP8>(s, j, b, s.nchunks - 1 - z);
    return;
  }
  if (z == s.nchunks) {  // the list's reuse decision
    if (threadIdx.x < 64) {
      const double C = group_cosine<T, D>((const T*)s.q, (const T*)s.reuse.q_prev, s.Hkv, G, b, j);
      if (threadIdx.x == 0) {
        const int list = b * s.Hkv + j;
        s.reuse.corrected[list] = (uint8_t)((s.reuse.first_step || C < s.reuse.tau) ? 1 : 0);
        if (s.reuse.similarity) s.reuse.similarity[list] = C;
      }
    }
    return;
  }
  if constexpr (sizeof(T) == 2)
    attn_bf16_block<D, P, S::WAVES, S::TPW, ROPE, 0, FP8>(a, G, j, b, z - s.nchunks - 1);
  else
    attn_f32_block<D, P, S::WAVES, S::TPW, ROPE>(a, G, j, b, z - s.nchunks - 1);
}

template <typename T, int D, int P, bool ROPE, bool FP8>
static hipError_t launch_co_r(const AttnArgs& a, SelectArgs s, int G, int prev_splits,
                              hipStream_t stream) {
  using S = FusedShape<T, P>;
  constexpr int PPB = S::WAVES * (64 / row_map<T, D>::LPR);  // pages per score block
  s.nchunks = (s.maxn + PPB - 1) / PPB;
  const dim3 grid(a.Hkv, a.nlists / a.Hkv, s.nchunks + 1 + prev_splits);
  const dim3 block(S::WAVES * 64);
  switch (G) {
    case 1: hipLaunchKernelGGL((spec_co_kernel<T, D, P, ROPE, 1, FP8>), grid, block, 0, stream, a, s); break;
    case 2: hipLaunchKernelGGL((spec_co_kernel<T, D, P, ROPE, 2, FP8>), grid, block, 0, stream, a, s); break;
    case 4: hipLaunchKernelGGL((spec_co_kernel<T, D, P, ROPE, 4, FP8>), grid, block, 0, stream, a, s); break;
    default: hipLaunchKernelGGL((spec_co_kernel<T, D, P, ROPE, 8, FP8>), grid, block, 0, stream, a, s); break;
  }
  return hipGetLastError();
}

template <typename T, int D, bool FP8 = false>
static hipError_t launch_co(int P, bool rope, const AttnArgs& a, const SelectArgs& s, int G,
                            int prev_splits, hipStream_t stream) {
  if constexpr (FP8) {  // no rotary gather on fp8 pools
    return P == 16 ? launch_co_r<T, D, 16, false, true>(a, s, G, prev_splits, stream)
                   : launch_co_r<T, D, 32, false, true>(a, s, G, prev_splits, stream);
  }
  if (P == 16) return rope ? launch_co_r<T, D, 16, true, false>(a, s, G, prev_splits, stream)
                           : launch_co_r<T, D, 16, false, false>(a, s, G, prev_splits, stream);
  return rope ? launch_co_r<T, D, 32, true, false>(a, s, G, prev_splits, stream)
              : launch_co_r<T, D, 32, false, false>(a, s, G, prev_splits, stream);
}

hipError_t launch_speculative_step(const LaunchKV& kv, const RopeArgs& rope, void* summ,
                                   const void* q, int k, int flags, float scale,
                                   const ReuseArgs& reuse, int32_t* sel_idx, int32_t* sel_cnt,
                                   void* out, float* lse, void* ws, hipStream_t stream) {
  float* scores = (float*)ws;
  void* attn_ws = (char*)ws + align256((size_t)kv.B * kv.Hkv * kv.maxp * sizeof(float));
  if (!fused_select_supported(kv, k)) {  // the two calls, serially
    hipError_t e = launch_score_topk(kv, rope, summ, q, k, flags, sel_idx, sel_cnt, scores, false,
                                     reuse, stream);
    if (e != hipSuccess) return e;
    return launch_attention(kv, rope, q, reuse.used_idx, reuse.used_cnt, k, scale,
                            step_pages_per_split(kv, k), out, lse,
                            attn_ws, stream);
  }
  const bool r = rope.page_row != nullptr;
  const SelectArgs s = select_args(kv, rope, summ, q, k, flags, nullptr, nullptr, scores, true, reuse);
  const AttnArgs prev = attn_args(kv, rope, q, reuse.prev_idx, reuse.prev_cnt, k, scale, FUSED_PPS,
                                  out, lse, attn_ws);
  const int prev_splits = reuse.first_step ? 0 : prev.nsplit;
  hipError_t e;
  if (kv.dtype == 2)
    e = kv.D == 64 ? launch_co<bf16_t, 64, true>(kv.P, r, prev, s, kv.G, prev_splits, stream)
                   : launch_co<bf16_t, 128, true>(kv.P, r, prev, s, kv.G, prev_splits, stream);
  else if (kv.dtype == 0)
    e = kv.D == 64 ? launch_co<float, 64>(kv.P, r, prev, s, kv.G, prev_splits, stream)
                   : launch_co<float, 128>(kv.P, r, prev, s, kv.G, prev_splits, stream);
  else
    e = kv.D == 64 ? launch_co<bf16_t, 64>(kv.P, r, prev, s, kv.G, prev_splits, stream)
                   : launch_co<bf16_t, 128>(kv.P, r, prev, s, kv.G, prev_splits, stream);
  if (e != hipSuccess) return e;
  AttnArgs f = attn_args(kv, rope, q, nullptr, nullptr, k, scale, FUSED_PPS, out, lse, attn_ws);
  f.scores = scores;
  f.sel_out = sel_idx;
  f.cnt_out = sel_cnt;
  f.reuse = reuse;
  return launch_fused_select(kv, f, r, stream);
}

}  // namespace kvsel
