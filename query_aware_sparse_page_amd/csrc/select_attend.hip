// kvsel_select_attend: the scores (score kernel), then the attention launch with the selection
// fused in (select_tiles: every block re-derives its list's top-k from the scores and keeps the
// pages of its own split), then the merge. The fused launch uses splits of FUSED_PPS pages (block
// shapes in kvsel_attn.h), the step's split below 64 lists (step_pages_per_split); with pages that
// end early (page_fill) it is a separate instantiation (FILL), taken at <= 4 keys per thread only.
// Other cases (many lists, a wide table, a k that needs larger splits; select_attend_fused) run
// the two separate calls' launches at the step's split instead.
#include "kvsel_attn.h"

namespace kvsel {

template <int D, int P, int WAVES, int TPW, bool ROPE, int C, bool FILL>
__global__ __launch_bounds__(WAVES * 64) void fused_bf16_kernel(AttnArgs a, int G) {
  // grid (Hkv, B, splits)
  attn_bf16_block<D, P, WAVES, TPW, ROPE, C, false, FILL>(a, G, blockIdx.x, blockIdx.y, blockIdx.z);
}

template <int D, int P, int WAVES, int TPW, int C, bool FILL>
__global__ __launch_bounds__(WAVES * 64) void fused_fp8_kernel(AttnArgs a, int G) {
  attn_bf16_block<D, P, WAVES, TPW, false, C, true, FILL>(a, G, blockIdx.x, blockIdx.y, blockIdx.z);
}

template <int D, int P, int WAVES, int TPW, bool ROPE, int C, bool FILL>
__global__ __launch_bounds__(WAVES * 64) void fused_f32_kernel(AttnArgs a, int G) {
  attn_f32_block<D, P, WAVES, TPW, ROPE, C, FILL>(a, G, blockIdx.x, blockIdx.y, blockIdx.z);
}

// Score keys per thread of the fused select (the block holds the whole table row in registers).
static int fused_keys_per_thread(const LaunchKV& kv) {
  const int nt = (kv.dtype != 0 && kv.P == 16) ? 128 : 256;  // FusedShape's threads
  const int c = (kv.maxn + nt - 1) / nt;
  return c <= 1 ? 1 : c <= 4 ? 4 : c <= 8 ? 8 : c <= 16 ? 16 : c <= 32 ? 32 : 0;
}

int step_pages_per_split(const LaunchKV& kv, int k) {
  return attention_pages_per_split(kv, k, kv.B * kv.Hkv < SELECT_ONE_LAUNCH_MIN_LISTS ? FUSED_PPS : 0);
}

static bool fused_shape(const LaunchKV& kv, int k) {
  return fused_keys_per_thread(kv) > 0 && step_pages_per_split(kv, k) == FUSED_PPS;
}

bool fused_select_supported(const LaunchKV& kv, int k) {
  return !kv.page_fill && fused_shape(kv, k);  // composed sequences: kvsel_select_attend only
}

// Every block of a list repeats the list's select, so the fused form pays where that select is
// cheap and the blocks are few: at most 4 keys per thread (tables of <= 1024 pages; 512 for bf16
// with P 16) and fewer lists than the one-launch selection takes. Measured with cold caches:
// 8 lists of 1024 pages 18.8 us against 20.2 us for the separate launches; 8 lists of 4096 pages
// 30.6 against 30.5; 128 lists of <= 512 pages 37.5 against 36.5.
bool select_attend_fused(const LaunchKV& kv, const RopeArgs&, int k) {
  return fused_shape(kv, k) && fused_keys_per_thread(kv) <= 4 &&
         kv.B * kv.Hkv < SELECT_ONE_LAUNCH_MIN_LISTS;
}

template <typename T, int D, int P, bool ROPE, int C, bool FILL>
static void launch_fused_c(const AttnArgs& a, int G, hipStream_t stream) {
  using S = FusedShape<T, P>;
  const dim3 grid(a.Hkv, a.nlists / a.Hkv, a.nsplit);
  const dim3 block(S::WAVES * 64);
  if constexpr (sizeof(T) == 1)
    hipLaunchKernelGGL((fused_fp8_kernel<D, P, S::WAVES, S::TPW, C, FILL>), grid, block, 0, stream, a, G);
  else if constexpr (sizeof(T) == 2)
    hipLaunchKernelGGL((fused_bf16_kernel<D, P, S::WAVES, S::TPW, ROPE, C, FILL>), grid, block, 0, stream, a, G);
  else
    hipLaunchKernelGGL((fused_f32_kernel<D, P, S::WAVES, S::TPW, ROPE, C, FILL>), grid, block, 0, stream, a, G);
}

template <typename T, int D, int P, bool ROPE>
static void launch_fused_r(int c, const AttnArgs& a, int G, hipStream_t stream) {
  if (a.page_fill) {  // c <= 4 (launch_fused_select checks)
    if (c == 1) launch_fused_c<T, D, P, ROPE, 1, true>(a, G, stream);
    else launch_fused_c<T, D, P, ROPE, 4, true>(a, G, stream);
    return;
  }
  switch (c) {
    case 1: launch_fused_c<T, D, P, ROPE, 1, false>(a, G, stream); break;
    case 4: launch_fused_c<T, D, P, ROPE, 4, false>(a, G, stream); break;
    case 8: launch_fused_c<T, D, P, ROPE, 8, false>(a, G, stream); break;
    case 16: launch_fused_c<T, D, P, ROPE, 16, false>(a, G, stream); break;
    default: launch_fused_c<T, D, P, ROPE, 32, false>(a, G, stream); break;
  }
}

template <typename T, int D>
static void launch_fused_p(int P, int c, const AttnArgs& a, int G, bool rope, hipStream_t stream) {
  if constexpr (sizeof(T) == 1) {  // fp8: no rotary gather
    if (P == 16) launch_fused_r<T, D, 16, false>(c, a, G, stream);
    else launch_fused_r<T, D, 32, false>(c, a, G, stream);
    return;
  }
  if (P == 16) {
    if (rope) launch_fused_r<T, D, 16, true>(c, a, G, stream);
    else launch_fused_r<T, D, 16, false>(c, a, G, stream);
  } else {
    if (rope) launch_fused_r<T, D, 32, true>(c, a, G, stream);
    else launch_fused_r<T, D, 32, false>(c, a, G, stream);
  }
}

hipError_t launch_fused_select(const LaunchKV& kv, const AttnArgs& a, bool rope,
                               hipStream_t stream) {
  const int c = fused_keys_per_thread(kv);
  if (a.page_fill && c > 4) return hipErrorInvalidValue;  // no such instantiation
  if (kv.dtype == 2) {
    if (kv.D == 64) launch_fused_p<fp8_t, 64>(kv.P, c, a, kv.G, false, stream);
    else launch_fused_p<fp8_t, 128>(kv.P, c, a, kv.G, false, stream);
  } else if (kv.dtype == 0) {
    if (kv.D == 64) launch_fused_p<float, 64>(kv.P, c, a, kv.G, rope, stream);
    else launch_fused_p<float, 128>(kv.P, c, a, kv.G, rope, stream);
  } else {
    if (kv.D == 64) launch_fused_p<bf16_t, 64>(kv.P, c, a, kv.G, rope, stream);
    else launch_fused_p<bf16_t, 128>(kv.P, c, a, kv.G, rope, stream);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_merge(kv, a, stream);
}

// The scores, then the partials of the step's split.
size_t select_attend_workspace(const LaunchKV& kv, int k) {
  return align256((size_t)kv.B * kv.Hkv * kv.maxp * sizeof(float)) +
         attention_workspace(kv, k, step_pages_per_split(kv, k));
}

hipError_t launch_select_attend(const LaunchKV& kv, const RopeArgs& rope, void* summ,
                                const void* q, int k, int flags, float scale, int32_t* sel_idx,
                                int32_t* sel_cnt, void* out, float* lse, void* ws,
                                hipStream_t stream) {
  float* scores = (float*)ws;
  void* attn_ws = (char*)ws + align256((size_t)kv.B * kv.Hkv * kv.maxp * sizeof(float));
  if (!select_attend_fused(kv, rope, k)) {
    hipError_t e = launch_score_topk(kv, rope, summ, q, k, flags, sel_idx, sel_cnt, scores, false,
                                     ReuseArgs{}, stream);
    if (e != hipSuccess) return e;
    return launch_attention(kv, rope, q, sel_idx, sel_cnt, k, scale, step_pages_per_split(kv, k),
                            out, lse, attn_ws, stream);
  }
  hipError_t e = launch_scores(kv, rope, summ, q, flags, scores, stream);
  if (e != hipSuccess) return e;
  AttnArgs a = attn_args(kv, rope, q, nullptr, nullptr, k, scale, FUSED_PPS, out, lse, attn_ws);
  a.scores = scores;
  a.sel_out = sel_idx;
  a.cnt_out = sel_cnt;
  return launch_fused_select(kv, a, rope.page_row != nullptr, stream);
}

}  // namespace kvsel
