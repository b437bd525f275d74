// Internal launch interface between the C ABI layer (kvsel_abi.hip) and the kernel files.
// Arguments reaching these launchers have been validated on the host.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvsel {

// Flattened, validated copy of a kvsel_paged_kv descriptor.
struct LaunchKV {
  int dtype;  // 0 = f32, 1 = bf16, 2 = fp8 E4M3 pools (q, summaries and outputs bf16)
  int B, Hq, Hkv, G, D, P, log2P, Npp;
  int maxp;  // page-table row width: the stride of the table, summaries and score rows
  int maxn;  // live pages at most (<= maxp): grids, key counts and the page bound of a sequence
  const void* k_pool;
  const void* v_pool;
  const int32_t* page_table;
  const int32_t* seq_lens;
  const float* k_scale;  // fp8 pools: [Npp][Hkv] per-tile scales (else null)
  const float* v_scale;
  const int32_t* page_fill;  // [Npp] valid slots of each physical page (composed sequences), or null
};

// Rotary table arguments passed to kernels by value; page_row == nullptr means "no rotation".
struct RopeArgs {
  const float* cos;
  const float* sin;
  const int32_t* page_row;
  int row_step;
  int per_seq;  // page_row by (sequence, logical page), row stride `stride`; else by physical page
  int stride;
};

// The page_row entry of logical page n (physical page p) of sequence b.
__host__ __device__ inline int rope_row_index(const RopeArgs& r, int b, int n, int p) {
  return r.per_seq ? b * r.stride + n : p;
}

// Per-pair inverse rotary frequencies theta^(-2i/D), i < D/2 <= 64 (kernel argument by value).
struct InvFreq {
  double v[64];
};

struct ReuseArgs {
  const void* q_prev;  // nullptr: no reuse decision
  const int32_t* prev_idx;
  const int32_t* prev_cnt;
  double tau;
  int first_step;
  int32_t* used_idx;
  int32_t* used_cnt;
  uint8_t* corrected;
  double* similarity;
};

hipError_t launch_summaries(const LaunchKV& kv, const RopeArgs& rope, int tail_only, void* summ,
                            hipStream_t stream);

// Blocks of the selection kernel per list (each block scores one chunk of pages).
int select_blocks_per_list(const LaunchKV& kv);

// scores_requested: the caller asked for the scores (else `scores` is workspace and the one-launch
// path may skip writing it).
hipError_t launch_score_topk(const LaunchKV& kv, const RopeArgs& rope, void* summ, const void* q,
                             int k, int flags, int32_t* sel_idx, int32_t* sel_cnt, float* scores,
                             bool scores_requested, const ReuseArgs& reuse, hipStream_t stream);

// Scores only (score kernel, with the optional tail refresh), into scores [B][Hkv][maxp].
hipError_t launch_scores(const LaunchKV& kv, const RopeArgs& rope, void* summ, const void* q,
                         int flags, float* scores, hipStream_t stream);

// Lists from which the selection runs as one launch (one block per list scores and selects;
// score_topk.hip) instead of the score and top-k launches.
constexpr int SELECT_ONE_LAUNCH_MIN_LISTS = 64;

// Selection + attention in one call: scores, then the attention launch with the selection fused
// in (when select_attend_fused), then the merge. Workspace: select_attend_workspace bytes.
// fused_select_supported: the fused launch exists for this shape (register-resident select of
// the table row, the default split); select_attend_fused: kvsel_select_attend also takes it.
bool fused_select_supported(const LaunchKV& kv, int k);
// Pages per split of the attention in kvsel_select_attend and kvsel_speculative_step: the fused
// launches' split below 64 lists, the default split from 64 lists on.
int step_pages_per_split(const LaunchKV& kv, int k);
bool select_attend_fused(const LaunchKV& kv, const RopeArgs& rope, int k);
size_t select_attend_workspace(const LaunchKV& kv, int k);
hipError_t launch_select_attend(const LaunchKV& kv, const RopeArgs& rope, void* summ,
                                const void* q, int k, int flags, float scale, int32_t* sel_idx,
                                int32_t* sel_cnt, void* out, float* lse, void* ws,
                                hipStream_t stream);

// The speculative step: scoring, the reuse decision and the attention over the previous pages
// in one launch, then the fused selection (corrected lists attended again) and the merge.
// Workspace: select_attend_workspace bytes.
hipError_t launch_speculative_step(const LaunchKV& kv, const RopeArgs& rope, void* summ,
                                   const void* q, int k, int flags, float scale,
                                   const ReuseArgs& reuse, int32_t* sel_idx, int32_t* sel_cnt,
                                   void* out, float* lse, void* ws, hipStream_t stream);

// Workspace of the attention for a given split size (bytes).
size_t attention_workspace(const LaunchKV& kv, int k, int pages_per_split);
int attention_pages_per_split(const LaunchKV& kv, int k, int requested);

hipError_t launch_attention(const LaunchKV& kv, const RopeArgs& rope, const void* q,
                            const int32_t* sel_idx, const int32_t* sel_cnt, int k, float scale,
                            int pages_per_split, void* out, float* lse, void* ws,
                            hipStream_t stream);

// Device-side free-page list of the append (ids == nullptr: the caller set the table entries).
struct FreePages {
  int32_t* ids;
  int32_t* count;
  int capacity;
};

// Decode-time append of one token per sequence (k_new / v_new [B][Hkv][D]), with the tail page's
// summary kept current when summ is non-null; writes seq_lens_out[b] = seq_lens[b] + 1.
hipError_t launch_append(const LaunchKV& kv, const void* k_new, const void* v_new, void* summ,
                         int32_t* seq_lens_out, const FreePages& free_pages, uint32_t* flags,
                         hipStream_t stream);

// fp8 quantization of every (physical page, KV head) tile of K (and of V when v_codes != null).
hipError_t launch_quantize(const LaunchKV& src, uint8_t* k_codes, float* k_scale, uint8_t* v_codes,
                           float* v_scale, hipStream_t stream);

// Device-side contract check; ORs KVSEL_CHECK_* bits into *flags.
hipError_t launch_check_inputs(const LaunchKV& kv, const int32_t* sel_idx, const int32_t* sel_cnt,
                               int k, uint32_t* flags, hipStream_t stream);

// Gather probe: n_chunks chunks of chunk_kib KiB (1..32, a power of two) at device addresses.
hipError_t launch_gather_probe(const uint64_t* addr, int n_chunks, int chunk_kib, uint32_t* sink,
                               hipStream_t stream);

hipError_t launch_rope_table(double theta, int D, int first_position, int n_rows, float* cos,
                             float* sin, hipStream_t stream);

hipError_t launch_rope_shift(const LaunchKV& kv, const RopeArgs& rope, void* k_out,
                             hipStream_t stream);

}  // namespace kvsel
