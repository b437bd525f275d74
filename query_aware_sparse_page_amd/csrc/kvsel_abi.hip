// C ABI of libkvsel.so: host-side validation, workspace sizing and dispatch to the kernels.
// Every check happens before anything is enqueued, so a failing call has no effect.
#include <hip/hip_runtime.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "../../include/kvsel.h"
#include "kvsel_internal.h"

using namespace kvsel;

// Scratch of kvsel_select_attend_static (scores and split partials): one copy per GPU, at its own
// address there. Host code never passes this name to a kernel (on the host it is a stand-in, not
// a device address); it uses the address looked up per device by static_scratch below.
static __device__ __align__(256) unsigned char scratch[KVSEL_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

kvsel_status check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KVSEL_ERR_DEVICE;
  int st = g_device_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return KVSEL_ERR_DEVICE;
    st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_device_state[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? KVSEL_OK : KVSEL_ERR_DEVICE;
}

int ilog2_exact(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return (1 << l) == x ? l : -1;
}

// Structural checks of a cache descriptor. need: bit 1 = V pool, bit 2 = page table + lengths.
kvsel_status flatten(const kvsel_paged_kv* kv, int need, LaunchKV* out) {
  if (!kv) return KVSEL_ERR_INVALID_ARGUMENT;
  if (kv->batch < 1 || kv->num_q_heads < 1 || kv->num_kv_heads < 1 || kv->head_dim < 1 ||
      kv->page_size < 1 || kv->num_phys_pages < 1 || kv->max_pages_per_seq < 1)
    return KVSEL_ERR_INVALID_ARGUMENT;
  if (kv->num_q_heads % kv->num_kv_heads != 0) return KVSEL_ERR_INVALID_ARGUMENT;
  if (!kv->k_pool) return KVSEL_ERR_INVALID_ARGUMENT;
  if ((need & 1) && !kv->v_pool) return KVSEL_ERR_INVALID_ARGUMENT;
  if ((need & 2) && (!kv->page_table || !kv->seq_lens)) return KVSEL_ERR_INVALID_ARGUMENT;
  if (kv->dtype != KVSEL_F32 && kv->dtype != KVSEL_BF16 && kv->dtype != KVSEL_FP8_E4M3)
    return KVSEL_ERR_UNSUPPORTED;
  if (kv->dtype == KVSEL_FP8_E4M3 && (!kv->k_scale || ((need & 1) && !kv->v_scale)))
    return KVSEL_ERR_INVALID_ARGUMENT;
  const int G = kv->num_q_heads / kv->num_kv_heads;
  if (kv->head_dim != 64 && kv->head_dim != 128) return KVSEL_ERR_UNSUPPORTED;
  if (kv->page_size != 16 && kv->page_size != 32) return KVSEL_ERR_UNSUPPORTED;
  if (G != 1 && G != 2 && G != 4 && G != 8) return KVSEL_ERR_UNSUPPORTED;
  // grid limits: sequences and page-range chunks index the second and third grid dimensions
  if (kv->batch > KVSEL_MAX_BATCH || kv->max_pages_per_seq > KVSEL_MAX_PAGES_PER_SEQ)
    return KVSEL_ERR_UNSUPPORTED;
  if (kv->max_seq_len < 0) return KVSEL_ERR_INVALID_ARGUMENT;
  out->dtype = kv->dtype == KVSEL_F32 ? 0 : kv->dtype == KVSEL_BF16 ? 1 : 2;
  out->B = kv->batch;
  out->Hq = kv->num_q_heads;
  out->Hkv = kv->num_kv_heads;
  out->G = G;
  out->D = kv->head_dim;
  out->P = kv->page_size;
  out->log2P = ilog2_exact(kv->page_size);
  out->Npp = kv->num_phys_pages;
  out->maxp = kv->max_pages_per_seq;
  out->maxn = kv->max_seq_len > 0
                  ? (int)std::min<long>(((long)kv->max_seq_len + kv->page_size - 1) / kv->page_size,
                                        (long)kv->max_pages_per_seq)
                  : kv->max_pages_per_seq;
  out->k_pool = kv->k_pool;
  out->v_pool = kv->v_pool;
  out->page_table = kv->page_table;
  out->seq_lens = kv->seq_lens;
  out->k_scale = out->dtype == 2 ? kv->k_scale : nullptr;
  out->v_scale = out->dtype == 2 ? kv->v_scale : nullptr;
  out->page_fill = kv->page_fill;
  return KVSEL_OK;
}

// A rotary argument of a call on cache f (fp8 caches take none).
kvsel_status flatten_rope(const kvsel_rope* rope, const LaunchKV& f, RopeArgs* out) {
  out->cos = nullptr;
  out->sin = nullptr;
  out->page_row = nullptr;
  out->row_step = 0;
  out->per_seq = 0;
  out->stride = f.maxp;
  if (!rope) return KVSEL_OK;
  if (f.dtype == 2) return KVSEL_ERR_UNSUPPORTED;
  if (!rope->cos || !rope->sin || !rope->page_row || rope->n_rows < 1) return KVSEL_ERR_INVALID_ARGUMENT;
  if (rope->row_step != 0 && rope->row_step != 1) return KVSEL_ERR_INVALID_ARGUMENT;
  out->cos = rope->cos;
  out->sin = rope->sin;
  out->page_row = rope->page_row;
  out->row_step = rope->row_step;
  out->per_seq = rope->per_sequence ? 1 : 0;
  return KVSEL_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Device address of `scratch` on the current device, looked up once per device with that device
// current (hipGetSymbolAddress) and kept.
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

kvsel_status static_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KVSEL_ERR_DEVICE;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KVSEL_ERR_DEVICE;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return KVSEL_OK;
}

// Room for the scores when the caller does not provide a score buffer.
size_t score_workspace(const LaunchKV& kv, bool with_scores) {
  return with_scores ? align256((size_t)kv.B * kv.Hkv * kv.maxp * sizeof(float)) : 0;
}

kvsel_status launch_status(hipError_t e) { return e == hipSuccess ? KVSEL_OK : KVSEL_ERR_LAUNCH; }

}  // namespace

extern "C" {

int32_t kvsel_abi_version(void) { return KVSEL_ABI_VERSION; }

const char* kvsel_status_str(kvsel_status status) {
  switch (status) {
    case KVSEL_OK: return "KVSEL_OK";
    case KVSEL_ERR_INVALID_ARGUMENT: return "KVSEL_ERR_INVALID_ARGUMENT: invalid argument";
    case KVSEL_ERR_UNSUPPORTED: return "KVSEL_ERR_UNSUPPORTED: shape or dtype without a kernel";
    case KVSEL_ERR_WORKSPACE: return "KVSEL_ERR_WORKSPACE: workspace missing or too small";
    case KVSEL_ERR_DEVICE: return "KVSEL_ERR_DEVICE: current device is not gfx950";
    case KVSEL_ERR_LAUNCH: return "KVSEL_ERR_LAUNCH: kernel launch failed";
    case KVSEL_ERR_SCRATCH:
      return "KVSEL_ERR_SCRATCH: the call needs more than the library's static scratch "
             "(KVSEL_STATIC_SCRATCH_BYTES); use the entry point that takes a workspace";
    default: return "KVSEL_ERR_UNKNOWN: unknown status code";
  }
}

size_t kvsel_workspace_bytes(const kvsel_paged_kv* kv, int32_t k, int32_t op,
                             int32_t pages_per_split) {
  LaunchKV f;
  if (k < 1 || flatten(kv, 0, &f) != KVSEL_OK) return 0;
  if (op == KVSEL_OP_SCORE_TOPK) return score_workspace(f, true);
  if (op == KVSEL_OP_ATTENTION) return attention_workspace(f, k, pages_per_split);
  if (op == KVSEL_OP_SELECT_ATTEND || op == KVSEL_OP_SPECULATIVE_STEP)
    return select_attend_workspace(f, k);
  return 0;
}

int32_t kvsel_step_pages_per_split(const kvsel_paged_kv* kv, int32_t k) {
  LaunchKV f;
  if (k < 1 || flatten(kv, 0, &f) != KVSEL_OK) return 0;
  return step_pages_per_split(f, k);
}

kvsel_status kvsel_build_summaries(const kvsel_paged_kv* kv, const kvsel_rope* rope,
                                   int32_t tail_only, void* summ, void* stream) {
  LaunchKV f;
  RopeArgs r;
  kvsel_status st = flatten(kv, 2, &f);
  if (st != KVSEL_OK) return st;
  if (!summ) return KVSEL_ERR_INVALID_ARGUMENT;
  if ((st = flatten_rope(rope, f, &r)) != KVSEL_OK) return st;
  if ((st = check_device()) != KVSEL_OK) return st;
  return launch_status(launch_summaries(f, r, tail_only ? 1 : 0, summ, (hipStream_t)stream));
}

kvsel_status kvsel_score_topk(const kvsel_paged_kv* kv, const kvsel_rope* rope, void* summ,
                              const void* q, int32_t k, int32_t flags, int32_t* sel_idx,
                              int32_t* sel_cnt, float* scores, const kvsel_reuse* reuse, void* ws,
                              size_t ws_bytes, void* stream) {
  LaunchKV f;
  RopeArgs r;
  kvsel_status st = flatten(kv, 2, &f);
  if (st != KVSEL_OK) return st;
  if (!summ || !q || !sel_idx || !sel_cnt || k < 1) return KVSEL_ERR_INVALID_ARGUMENT;
  if (flags & ~KVSEL_SCORE_REFRESH_TAIL) return KVSEL_ERR_INVALID_ARGUMENT;
  if ((st = flatten_rope(rope, f, &r)) != KVSEL_OK) return st;
  ReuseArgs ra;
  memset(&ra, 0, sizeof(ra));
  if (reuse) {
    if (!reuse->q_prev || !reuse->prev_idx || !reuse->prev_cnt || !reuse->used_idx ||
        !reuse->used_cnt || !reuse->corrected)
      return KVSEL_ERR_INVALID_ARGUMENT;
    ra.q_prev = reuse->q_prev;
    ra.prev_idx = reuse->prev_idx;
    ra.prev_cnt = reuse->prev_cnt;
    ra.tau = reuse->tau;
    ra.first_step = reuse->first_step;
    ra.used_idx = reuse->used_idx;
    ra.used_cnt = reuse->used_cnt;
    ra.corrected = reuse->corrected;
    ra.similarity = reuse->similarity;
  }
  const bool requested = scores != nullptr;
  if (!scores) {
    if (!ws || ws_bytes < score_workspace(f, true)) return KVSEL_ERR_WORKSPACE;
    scores = (float*)ws;
  }
  if ((st = check_device()) != KVSEL_OK) return st;
  return launch_status(launch_score_topk(f, r, summ, q, k, flags, sel_idx, sel_cnt, scores,
                                         requested, ra, (hipStream_t)stream));
}

kvsel_status kvsel_sparse_decode_attn(const kvsel_paged_kv* kv, const kvsel_rope* rope,
                                      const void* q, const int32_t* sel_idx,
                                      const int32_t* sel_cnt, int32_t k, float scale,
                                      int32_t pages_per_split, void* out, float* lse, void* ws,
                                      size_t ws_bytes, void* stream) {
  LaunchKV f;
  RopeArgs r;
  kvsel_status st = flatten(kv, 3, &f);
  if (st != KVSEL_OK) return st;
  if (!q || !sel_idx || !sel_cnt || !out || k < 1 || pages_per_split < 0)
    return KVSEL_ERR_INVALID_ARGUMENT;
  if ((st = flatten_rope(rope, f, &r)) != KVSEL_OK) return st;
  if (attention_pages_per_split(f, k, pages_per_split) <= 0) return KVSEL_ERR_UNSUPPORTED;
  const size_t need = attention_workspace(f, k, pages_per_split);
  if (need > 0 && (!ws || ws_bytes < need)) return KVSEL_ERR_WORKSPACE;
  if ((st = check_device()) != KVSEL_OK) return st;
  return launch_status(launch_attention(f, r, q, sel_idx, sel_cnt, k, scale, pages_per_split, out,
                                        lse, ws, (hipStream_t)stream));
}

kvsel_status kvsel_select_attend(const kvsel_paged_kv* kv, const kvsel_rope* rope, void* summ,
                                 const void* q, int32_t k, int32_t flags, float scale,
                                 int32_t* sel_idx, int32_t* sel_cnt, void* out, float* lse,
                                 void* ws, size_t ws_bytes, void* stream) {
  LaunchKV f;
  RopeArgs r;
  kvsel_status st = flatten(kv, 3, &f);
  if (st != KVSEL_OK) return st;
  if (!summ || !q || !sel_idx || !sel_cnt || !out || k < 1) return KVSEL_ERR_INVALID_ARGUMENT;
  if (flags & ~KVSEL_SCORE_REFRESH_TAIL) return KVSEL_ERR_INVALID_ARGUMENT;
  if ((st = flatten_rope(rope, f, &r)) != KVSEL_OK) return st;
  if (step_pages_per_split(f, k) <= 0) return KVSEL_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < select_attend_workspace(f, k)) return KVSEL_ERR_WORKSPACE;
  if ((st = check_device()) != KVSEL_OK) return st;
  return launch_status(launch_select_attend(f, r, summ, q, k, flags, scale, sel_idx, sel_cnt, out,
                                            lse, ws, (hipStream_t)stream));
}

kvsel_status kvsel_select_attend_static(const kvsel_paged_kv* kv, const kvsel_rope* rope,
                                        void* summ, const void* q, int32_t k, int32_t flags,
                                        float scale, int32_t* sel_idx, int32_t* sel_cnt, void* out,
                                        float* lse, void* stream) {
  LaunchKV f;
  RopeArgs r;
  kvsel_status st = flatten(kv, 3, &f);
  if (st != KVSEL_OK) return st;
  if (!summ || !q || !sel_idx || !sel_cnt || !out || k < 1) return KVSEL_ERR_INVALID_ARGUMENT;
  if (flags & ~KVSEL_SCORE_REFRESH_TAIL) return KVSEL_ERR_INVALID_ARGUMENT;
  if ((st = flatten_rope(rope, f, &r)) != KVSEL_OK) return st;
  if (step_pages_per_split(f, k) <= 0) return KVSEL_ERR_UNSUPPORTED;
  if (select_attend_workspace(f, k) > (size_t)KVSEL_STATIC_SCRATCH_BYTES) return KVSEL_ERR_SCRATCH;
  if ((st = check_device()) != KVSEL_OK) return st;
  void* ws = nullptr;
  if ((st = static_scratch(&ws)) != KVSEL_OK) return st;
  return launch_status(launch_select_attend(f, r, summ, q, k, flags, scale, sel_idx, sel_cnt, out,
                                            lse, ws, (hipStream_t)stream));
}

kvsel_status kvsel_speculative_step(const kvsel_paged_kv* kv, const kvsel_rope* rope, void* summ,
                                    const void* q, int32_t k, int32_t flags, float scale,
                                    const kvsel_reuse* reuse, int32_t* sel_idx, int32_t* sel_cnt,
                                    void* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  LaunchKV f;
  RopeArgs r;
  kvsel_status st = flatten(kv, 3, &f);
  if (st != KVSEL_OK) return st;
  if (!summ || !q || !sel_idx || !sel_cnt || !out || k < 1 || !reuse) return KVSEL_ERR_INVALID_ARGUMENT;
  if (!reuse->q_prev || !reuse->prev_idx || !reuse->prev_cnt || !reuse->used_idx ||
      !reuse->used_cnt || !reuse->corrected)
    return KVSEL_ERR_INVALID_ARGUMENT;
  if (flags & ~KVSEL_SCORE_REFRESH_TAIL) return KVSEL_ERR_INVALID_ARGUMENT;
  if ((st = flatten_rope(rope, f, &r)) != KVSEL_OK) return st;
  if (step_pages_per_split(f, k) <= 0) return KVSEL_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < select_attend_workspace(f, k)) return KVSEL_ERR_WORKSPACE;
  ReuseArgs ra;
  memset(&ra, 0, sizeof(ra));
  ra.q_prev = reuse->q_prev;
  ra.prev_idx = reuse->prev_idx;
  ra.prev_cnt = reuse->prev_cnt;
  ra.tau = reuse->tau;
  ra.first_step = reuse->first_step;
  ra.used_idx = reuse->used_idx;
  ra.used_cnt = reuse->used_cnt;
  ra.corrected = reuse->corrected;
  ra.similarity = reuse->similarity;
  if ((st = check_device()) != KVSEL_OK) return st;
  return launch_status(launch_speculative_step(f, r, summ, q, k, flags, scale, ra, sel_idx,
                                               sel_cnt, out, lse, ws, (hipStream_t)stream));
}

kvsel_status kvsel_check_inputs(const kvsel_paged_kv* kv, const int32_t* sel_idx,
                                const int32_t* sel_cnt, int32_t k, uint32_t* flags, void* stream) {
  LaunchKV f;
  kvsel_status st = flatten(kv, 2, &f);
  if (st != KVSEL_OK) return st;
  if (!flags || (sel_idx && (!sel_cnt || k < 1))) return KVSEL_ERR_INVALID_ARGUMENT;
  if ((st = check_device()) != KVSEL_OK) return st;
  return launch_status(launch_check_inputs(f, sel_idx, sel_cnt, k, flags, (hipStream_t)stream));
}

kvsel_status kvsel_append_kv(const kvsel_paged_kv* kv, const void* k_new, const void* v_new,
                             void* summ, int32_t* seq_lens_out,
                             const kvsel_free_pages* free_pages, uint32_t* flags, void* stream) {
  LaunchKV f;
  kvsel_status st = flatten(kv, 3, &f);
  if (st != KVSEL_OK) return st;
  if (f.dtype == 2) return KVSEL_ERR_UNSUPPORTED;  // an fp8 page's scale is fixed at quantization
  if (!k_new || !v_new || !seq_lens_out) return KVSEL_ERR_INVALID_ARGUMENT;
  FreePages fp{nullptr, nullptr, 0};
  if (free_pages) {
    if (!free_pages->ids || !free_pages->count || free_pages->capacity < 1)
      return KVSEL_ERR_INVALID_ARGUMENT;
    fp = FreePages{free_pages->ids, free_pages->count, free_pages->capacity};
  }
  if ((st = check_device()) != KVSEL_OK) return st;
  return launch_status(launch_append(f, k_new, v_new, summ, seq_lens_out, fp, flags,
                                     (hipStream_t)stream));
}

kvsel_status kvsel_quantize_pages(const kvsel_paged_kv* src, uint8_t* k_codes, float* k_scale,
                                  uint8_t* v_codes, float* v_scale, void* stream) {
  LaunchKV f;
  const bool with_v = v_codes || v_scale;
  kvsel_status st = flatten(src, with_v ? 1 : 0, &f);
  if (st != KVSEL_OK) return st;
  if (f.dtype == 2) return KVSEL_ERR_UNSUPPORTED;  // the source is an f32 or bf16 cache
  if (!k_codes || !k_scale || (with_v && (!v_codes || !v_scale))) return KVSEL_ERR_INVALID_ARGUMENT;
  if ((st = check_device()) != KVSEL_OK) return st;
  return launch_status(
      launch_quantize(f, k_codes, k_scale, v_codes, v_scale, (hipStream_t)stream));
}

kvsel_status kvsel_gather_probe(const uint64_t* chunk_addr, int32_t n_chunks, int32_t chunk_bytes,
                                uint32_t* sink, void* stream) {
  if (!chunk_addr || !sink || n_chunks < 1 || n_chunks > (1 << 26)) return KVSEL_ERR_INVALID_ARGUMENT;
  const int kib = chunk_bytes / 1024;
  if (chunk_bytes % 1024 || kib < 1 || kib > 32 || (kib & (kib - 1))) return KVSEL_ERR_INVALID_ARGUMENT;
  kvsel_status st = check_device();
  if (st != KVSEL_OK) return st;
  return launch_status(launch_gather_probe(chunk_addr, n_chunks, kib, sink, (hipStream_t)stream));
}

kvsel_status kvsel_rope_table(double theta, int32_t head_dim, int32_t first_position,
                              int32_t n_rows, float* cos_t, float* sin_t, void* stream) {
  if (!cos_t || !sin_t || n_rows < 1 || head_dim < 2 || head_dim > 128 || (head_dim & 1) ||
      !(theta > 0.0))
    return KVSEL_ERR_INVALID_ARGUMENT;
  kvsel_status st = check_device();
  if (st != KVSEL_OK) return st;
  return launch_status(
      launch_rope_table(theta, head_dim, first_position, n_rows, cos_t, sin_t, (hipStream_t)stream));
}

kvsel_status kvsel_rope_shift(const kvsel_paged_kv* kv, const kvsel_rope* rope, void* k_out,
                              void* stream) {
  LaunchKV f;
  RopeArgs r;
  kvsel_status st = flatten(kv, 0, &f);
  if (st != KVSEL_OK) return st;
  if (!rope || !k_out) return KVSEL_ERR_INVALID_ARGUMENT;
  if ((st = flatten_rope(rope, f, &r)) != KVSEL_OK) return st;
  if (r.per_seq) return KVSEL_ERR_UNSUPPORTED;  // a shared physical page has one rotation
  if ((st = check_device()) != KVSEL_OK) return st;
  return launch_status(launch_rope_shift(f, r, k_out, (hipStream_t)stream));
}

}  // extern "C"
