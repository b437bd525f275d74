// Decode-time append: each sequence's new token key and value go into the tail page of the paged
// cache, and that page's summary is kept current without re-reading the page.
//
// One block per sequence, one wave per KV head (up to 16 waves; more heads in turn): LPR lanes
// carry the head's D channels as 16-byte slices. The key row is one 16-byte store per lane
// (token-major K pages); the value is a column of the channel-major V page (one element per
// channel, at stride P), written element by element as raw bits. The summary of a page that the
// token opens is the key itself (lo = hi); otherwise lo = min(lo, key), hi = max(hi, key) over
// the stored row -- exactly the rebuild of the page's valid keys when the stored summary covered
// the earlier ones (min and max are exact). The sequence length is read by every thread first
// and written once after a barrier, so the output may be the length array itself.
#include "kvsel_device.h"
#include "kvsel_internal.h"

namespace kvsel {

constexpr int APPEND_MAX_WAVES = 16;

struct AppendArgs {
  void* k_pool;
  void* v_pool;
  const int32_t* page_table;
  const int32_t* seq_lens;
  int32_t* seq_lens_out;
  const void* k_new;  // [B][Hkv][D]
  const void* v_new;  // [B][Hkv][D]
  void* summ;         // [B][Hkv][maxp][2][D], may be null
  uint32_t* flags;    // may be null
  int32_t* table_w;   // the page table, written when a page is taken from the free list
  FreePages free;     // free.ids == nullptr: the caller set the table entries
  int Hkv, P, maxp, Npp;
};

// Pop one page id off the free list for sequence b's logical page n (one thread): returns the
// page, or -1 with the reason ORed into the flags (an empty list is left as it was).
__device__ __forceinline__ int take_free_page(const AppendArgs& a, int b, int n) {
  const int top = atomicSub(a.free.count, 1);
  if (top <= 0) {
    atomicAdd(a.free.count, 1);  // the list was empty: give the count back
    if (a.flags) atomicOr(a.flags, 8u);  // KVSEL_CHECK_NO_FREE_PAGE
    return -1;
  }
  const int id = top <= a.free.capacity ? a.free.ids[top - 1] : -1;
  if (id < 0 || id >= a.Npp) {
    if (a.flags) atomicOr(a.flags, 2u);  // KVSEL_CHECK_PAGE_ID
    return -1;
  }
  a.table_w[(size_t)b * a.maxp + n] = id;
  return id;
}

// The raw element bits of one 16-byte slice, one element at a time.
template <typename T>
__device__ __forceinline__ void store_slice_column(T* base, size_t stride, const uint4& v);
template <>
__device__ __forceinline__ void store_slice_column<float>(float* base, size_t stride, const uint4& v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) reinterpret_cast<uint32_t*>(base)[e * stride] = w[e];
}
template <>
__device__ __forceinline__ void store_slice_column<bf16_t>(bf16_t* base, size_t stride,
                                                           const uint4& v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 8; ++e)
    reinterpret_cast<uint16_t*>(base)[e * stride] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
}

// Block of min(Hkv, APPEND_MAX_WAVES) waves: wave w takes KV heads w, w + waves, ... The first
// head's new rows are requested before the length (their addresses do not depend on it), and
// the page-table entry and stored summary rows together right after it, so one memory round trip
// follows the length's.
template <typename T, int D>
__global__ __launch_bounds__(APPEND_MAX_WAVES * 64) void append_kernel(AppendArgs a) {
  using M = row_map<T, D>;
  constexpr int VEC = M::VEC, LPR = M::LPR;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int NW = blockDim.x >> 6;
  const int c0 = lane * VEC;
  const bool row_lane = lane < LPR;
  uint4 kv = make_uint4(0, 0, 0, 0), vv = kv;
  if (row_lane && w < a.Hkv) {
    const size_t in = ((size_t)b * a.Hkv + w) * D + c0;
    kv = load16((const T*)a.k_new + in);
    vv = load16((const T*)a.v_new + in);
  }
  const int L = a.seq_lens[b];
  bool ok = L >= 0 && (long)L < (long)a.maxp * a.P;  // room for one more token
  if (!ok && a.flags && tid == 0) atomicOr(a.flags, 1u);  // KVSEL_CHECK_SEQ_LEN
  if (ok) {
    const int n = L / a.P, slot = L - n * a.P;
    int p;
    if (slot == 0 && a.free.ids) {  // block-uniform: the token opens a page from the free list
      __shared__ int s_page;
      if (tid == 0) s_page = take_free_page(a, b, n);
      __syncthreads();
      p = s_page;
      ok = p >= 0;
    } else {
      // the caller's allocator set this entry; clamp like every reader
      p = min(max(a.page_table[(size_t)b * a.maxp + n], 0), a.Npp - 1);
    }
    for (int j = w; ok && j < a.Hkv; j += NW) {
      if (!row_lane) continue;
      if (j != w) {
        const size_t in = ((size_t)b * a.Hkv + j) * D + c0;
        kv = load16((const T*)a.k_new + in);
        vv = load16((const T*)a.v_new + in);
      }
      T* row = a.summ ? (T*)a.summ + (((size_t)b * a.Hkv + j) * a.maxp + n) * 2 * D + c0 : nullptr;
      uint4 lo = kv, hi = kv;
      if (row && slot > 0) {
        float k[VEC], l0[VEC], h0[VEC];
        const uint4 lraw = load16(row), hraw = load16(row + D);
        unpack<T>(kv, k);
        unpack<T>(lraw, l0);
        unpack<T>(hraw, h0);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          l0[e] = tmin(l0[e], k[e]);
          h0[e] = tmax(h0[e], k[e]);
        }
        lo = pack<T>(l0);
        hi = pack<T>(h0);
      }
      store16((T*)a.k_pool + (((size_t)p * a.Hkv + j) * a.P + slot) * D + c0, kv);
      store_slice_column<T>((T*)a.v_pool + (((size_t)p * a.Hkv + j) * D + c0) * a.P + slot,
                            (size_t)a.P, vv);
      if (row) {
        store16(row, lo);
        store16(row + D, hi);
      }
    }
  }
  __syncthreads();  // every thread has read the length before it changes
  if (ok && tid == 0) a.seq_lens_out[b] = L + 1;
}

template <typename T>
static void launch_append_t(int D, const AppendArgs& a, int B, hipStream_t stream) {
  const dim3 block(64 * (a.Hkv < APPEND_MAX_WAVES ? a.Hkv : APPEND_MAX_WAVES));
  if (D == 64)
    hipLaunchKernelGGL((append_kernel<T, 64>), dim3(B), block, 0, stream, a);
  else
    hipLaunchKernelGGL((append_kernel<T, 128>), dim3(B), block, 0, stream, a);
}

hipError_t launch_append(const LaunchKV& kv, const void* k_new, const void* v_new, void* summ,
                         int32_t* seq_lens_out, const FreePages& free_pages, uint32_t* flags,
                         hipStream_t stream) {
  AppendArgs a;
  a.k_pool = const_cast<void*>(kv.k_pool);
  a.v_pool = const_cast<void*>(kv.v_pool);
  a.page_table = kv.page_table;
  a.seq_lens = kv.seq_lens;
  a.seq_lens_out = seq_lens_out;
  a.k_new = k_new;
  a.v_new = v_new;
  a.summ = summ;
  a.flags = flags;
  a.table_w = const_cast<int32_t*>(kv.page_table);
  a.free = free_pages;
  a.Hkv = kv.Hkv;
  a.P = kv.P;
  a.maxp = kv.maxp;
  a.Npp = kv.Npp;
  if (kv.dtype == 0) launch_append_t<float>(kv.D, a, kv.B, stream);
  else launch_append_t<bf16_t>(kv.D, a, kv.B, stream);
  return hipGetLastError();
}

}  // namespace kvsel
