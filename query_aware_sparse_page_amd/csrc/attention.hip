// Sparse paged decode attention: the split launch over the selected pages (one block per
// (KV head, sequence, split), body attn_bf16_block / attn_f32_block) and the log-sum-exp merge
// of the splits in a second launch. The kernel design (tiles, MFMA layouts, softmax, partials)
// is described in kvsel_attn.h.
#include <type_traits>

#include "kvsel_attn.h"

namespace kvsel {

// FILL: pages that end early (page_fill set), a separate instantiation.
template <int D, int P, int WAVES, int TPW, bool ROPE, bool FILL = false>
__global__ __launch_bounds__(WAVES * 64) void attn_bf16_kernel(AttnArgs a, int G) {
  // grid (Hkv, B, splits)
  attn_bf16_block<D, P, WAVES, TPW, ROPE, 0, false, FILL>(a, G, blockIdx.x, blockIdx.y, blockIdx.z);
}

// fp8 pools (E4M3 codes, per-tile scales), decoded to bf16 in registers; no rotary gather.
template <int D, int P, int WAVES, int TPW, bool FILL = false>
__global__ __launch_bounds__(WAVES * 64) void attn_fp8_kernel(AttnArgs a, int G) {
  attn_bf16_block<D, P, WAVES, TPW, false, 0, true, FILL>(a, G, blockIdx.x, blockIdx.y, blockIdx.z);
}

template <int D, int P, int WAVES, int TPW, bool ROPE, bool FILL = false>
__global__ __launch_bounds__(WAVES * 64) void attn_f32_kernel(AttnArgs a, int G) {
  attn_f32_block<D, P, WAVES, TPW, ROPE, 0, FILL>(a, G, blockIdx.x, blockIdx.y, blockIdx.z);
}

// ------------------------------------------------------------------------------------------
// merge: one block per (list, query head of the group), one thread per channel.
//
// attn_merge_kernel (up to 64 splits): every thread loads its channel's accumulator of each split
// (MC >= nsplit loads, clamped indices, block-uniform row bases) and lane s of every wave loads
// split s's (m, l, lu), all in one memory round trip. Each wave then forms the split weights
// lane-parallel: M = max m_s and the sums of l_s and lu_s weighted by e^(m_s - M) are wave-wide
// reductions on DPP and the lane swaps, and the weights reach the wave's lanes through LDS, so no
// block barrier is needed. Splits are combined in split order, as in the wide form.
// attn_merge_wide_kernel (more splits): the (m, l, lu) of every split through LDS, accumulators in
// rounds of MERGE_CHUNK splits.
// ------------------------------------------------------------------------------------------
constexpr int MERGE_CHUNK = 32;

template <typename T, int D, int MC>
__global__ __launch_bounds__(D) void attn_merge_kernel(AttnArgs a, int G) {
  static_assert(MC <= 64, "one split per lane");
  const float NEG_INF = __int_as_float(0xff800000);
  // grid (Hkv, G, B): KV heads vary fastest, as in the attention grid, so a list's merge blocks
  // are dispatched to the XCD that ran its splits (round-robin placement)
  const int j = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int list = b * a.Hkv + j;
  const int d = threadIdx.x, lane = d & 63, w = d >> 6;
  const int Hq = a.Hkv * G;
  const int ns = a.nsplit;
  const float4* ml = a.part_ml + (size_t)list * ns * G + g;
  const float* pa = a.part_acc + ((size_t)list * ns * G + g) * D;  // block-uniform base
  const int GD = G * D;
  const float4 mv = ml[(size_t)min(lane, ns - 1) * G];
  float v[MC];
#pragma unroll
  for (int u = 0; u < MC; ++u) v[u] = (pa + min(u, ns - 1) * GD)[d];
  __builtin_amdgcn_sched_barrier(0);
  const bool ok = lane < ns && mv.x != NEG_INF;  // a split with no valid token has m = -inf
  const float M = wave_allreduce_f32(ok ? mv.x : NEG_INF, [](float x, float y) { return fmaxf(x, y); });
  const float f = ok ? __expf(mv.x - M) : 0.0f;
  const float L = wave_allreduce_f32(ok ? mv.y * f : 0.0f, [](float x, float y) { return x + y; });
  const float LU = wave_allreduce_f32(ok ? mv.z * f : 0.0f, [](float x, float y) { return x + y; });
  __shared__ float s_f[D / 64][64];  // this wave's split weights (lane s: split s)
  s_f[w][lane] = f;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float A = 0.0f;
#pragma unroll
  for (int u = 0; u < MC; ++u) A = fmaf(v[u], s_f[w][u], A);  // weight 0 past the last split
  const size_t o = ((size_t)b * Hq + j * G + g) * D + d;
  store_elem<T>((T*)a.out, o, M == NEG_INF ? 0.0f : A / L);
  if (d == 0 && a.lse) a.lse[(size_t)b * Hq + j * G + g] = M == NEG_INF ? NEG_INF : M + logf(LU);
}

template <typename T, int D>
__global__ __launch_bounds__(D) void attn_merge_wide_kernel(AttnArgs a, int G) {
  const float NEG_INF = __int_as_float(0xff800000);
  const int j = blockIdx.x, g = blockIdx.y, b = blockIdx.z;  // grid (Hkv, G, B)
  const int list = b * a.Hkv + j;
  const int d = threadIdx.x;
  const int Hq = a.Hkv * G;
  const int ns = a.nsplit;
  __shared__ float s_m[ATT_MAX_SPLITS], s_l[ATT_MAX_SPLITS], s_lu[ATT_MAX_SPLITS];
  const float4* ml = a.part_ml + (size_t)list * ns * G + g;
  const float* pa = a.part_acc + ((size_t)list * ns * G + g) * D;  // block-uniform base
  const int GD = G * D;
  // one round of unconditional loads with clamped indices (a conditional load would make the
  // compiler wait for each one before the next)
  const float4 mv = ml[min(d, ns - 1) * G];
  float v[MERGE_CHUNK];
#pragma unroll
  for (int u = 0; u < MERGE_CHUNK; ++u) v[u] = (pa + min(u, ns - 1) * GD)[d];
  __builtin_amdgcn_sched_barrier(0);
  if (d < ns) {
    s_m[d] = mv.x;
    s_l[d] = mv.y;
    s_lu[d] = mv.z;
  }
  for (int s = d + D; s < ns; s += D) {  // more splits than threads
    const float4 x = ml[(size_t)s * G];
    s_m[s] = x.x;
    s_l[s] = x.y;
    s_lu[s] = x.z;
  }
  __syncthreads();
  float M = NEG_INF;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, s_m[s]);
  const size_t o = ((size_t)b * Hq + j * G + g) * D + d;
  if (M == NEG_INF) {
    store_elem<T>((T*)a.out, o, 0.0f);
    if (d == 0 && a.lse) a.lse[(size_t)b * Hq + j * G + g] = NEG_INF;
    return;
  }
  float L = 0.0f, LU = 0.0f, A = 0.0f;
  for (int s0 = 0; s0 < ns; s0 += MERGE_CHUNK) {
    if (s0 > 0) {
#pragma unroll
      for (int u = 0; u < MERGE_CHUNK; ++u) v[u] = (pa + min(s0 + u, ns - 1) * GD)[d];
    }
#pragma unroll
    for (int u = 0; u < MERGE_CHUNK; ++u) {
      const int s = s0 + u;
      if (s < ns && s_m[s] != NEG_INF) {
        const float f = __expf(s_m[s] - M);
        L = fmaf(s_l[s], f, L);
        LU = fmaf(s_lu[s], f, LU);
        A = fmaf(v[u], f, A);
      }
    }
  }
  store_elem<T>((T*)a.out, o, A / L);
  if (d == 0 && a.lse) a.lse[(size_t)b * Hq + j * G + g] = M + logf(LU);
}

// ------------------------------------------------------------------------------------------
// host side
// ------------------------------------------------------------------------------------------

// Tiles per split for a request of pps pages; 0 when the split size has no kernel. A split is
// WAVES * TPW tiles with (WAVES, TPW) in {(1,1), (2,1), (4,1), (4,2)}.
static int tiles_for(const LaunchKV& kv, int pps) {
  const int tt = kv.dtype == 0 ? 16 : 32;
  const int rows = pps * kv.P;
  if (rows % tt) return 0;
  const int tiles = rows / tt;
  return (tiles == 1 || tiles == 2 || tiles == 4 || tiles == 8) ? tiles : 0;
}

int attention_pages_per_split(const LaunchKV& kv, int k, int requested) {
  // default: below 64 lists a call is latency-bound, and the split that puts about one block on
  // each of the 256 CUs measured best (2 pages when lists x k/2 <= 256: one 32K sequence at k 64,
  // 6.82 against 7.80 us for 4 pages with cold caches; else 4: one 128K sequence at k 128, 8.60
  // against 9.21 us for 2 pages); from 64 lists on the call is bandwidth-bound, and 8 pages halve
  // the partials and the merge's loads
  const int nl = kv.B * kv.Hkv;
  const int want = requested > 0 ? requested : nl >= 64 ? 8 : (nl * ((k + 1) / 2) <= 256 ? 2 : 4);
  int pps = 0;
  // largest supported split not above the request, else the smallest supported one
  for (int p = want; p >= 1 && !pps; --p)
    if (tiles_for(kv, p)) pps = p;
  for (int p = want + 1; p <= 64 && !pps; ++p)
    if (tiles_for(kv, p)) pps = p;
  // at most ATT_MAX_SPLITS splits per list
  while (pps && (k + pps - 1) / pps > ATT_MAX_SPLITS) {
    int next = 0;
    for (int p = pps + 1; p <= 64 && !next; ++p)
      if (tiles_for(kv, p)) next = p;
    pps = next;
  }
  return pps;
}

size_t attention_workspace(const LaunchKV& kv, int k, int pages_per_split) {
  const int pps = attention_pages_per_split(kv, k, pages_per_split);
  if (pps <= 0) return 0;
  const size_t nsplit = (size_t)((k + pps - 1) / pps);
  if (nsplit <= 1) return 0;
  const size_t parts = (size_t)kv.B * kv.Hkv * nsplit * kv.G;
  return align256(parts * kv.D * sizeof(float)) + parts * sizeof(float4);
}

template <typename T, int D, int P, int WAVES, int TPW, bool FILL>
static void launch_split_f(const AttnArgs& a, int G, bool rope, hipStream_t stream) {
  const dim3 grid(a.Hkv, a.nlists / a.Hkv, a.nsplit);
  const dim3 block(WAVES * 64);
  if constexpr (sizeof(T) == 1) {
    hipLaunchKernelGGL((attn_fp8_kernel<D, P, WAVES, TPW, FILL>), grid, block, 0, stream, a, G);
  } else if constexpr (sizeof(T) == 2) {
    if (rope) hipLaunchKernelGGL((attn_bf16_kernel<D, P, WAVES, TPW, true, FILL>), grid, block, 0, stream, a, G);
    else hipLaunchKernelGGL((attn_bf16_kernel<D, P, WAVES, TPW, false, FILL>), grid, block, 0, stream, a, G);
  } else {
    if (rope) hipLaunchKernelGGL((attn_f32_kernel<D, P, WAVES, TPW, true, FILL>), grid, block, 0, stream, a, G);
    else hipLaunchKernelGGL((attn_f32_kernel<D, P, WAVES, TPW, false, FILL>), grid, block, 0, stream, a, G);
  }
}

template <typename T, int D, int P, int WAVES, int TPW>
static void launch_split(const AttnArgs& a, int G, bool rope, hipStream_t stream) {
  if (a.page_fill) launch_split_f<T, D, P, WAVES, TPW, true>(a, G, rope, stream);
  else launch_split_f<T, D, P, WAVES, TPW, false>(a, G, rope, stream);
}

// parts: 1 = the split launch, 2 = the merge launch (when there is more than one split)
template <typename T, int D, int P>
static hipError_t launch_tiles(int tiles, const AttnArgs& a, int G, bool rope, int parts,
                               hipStream_t stream) {
  if (parts & 1) {
    switch (tiles) {
      case 1: launch_split<T, D, P, 1, 1>(a, G, rope, stream); break;
      case 2: launch_split<T, D, P, 2, 1>(a, G, rope, stream); break;
      case 4: launch_split<T, D, P, 4, 1>(a, G, rope, stream); break;
      default: launch_split<T, D, P, 4, 2>(a, G, rope, stream); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!(parts & 2) || a.nsplit == 1) return hipSuccess;
  using OT = std::conditional_t<sizeof(T) == 1, bf16_t, T>;  // fp8 pools: bf16 outputs
  const dim3 grid(a.Hkv, G, a.nlists / a.Hkv);
  if (a.nsplit <= 8)
    hipLaunchKernelGGL((attn_merge_kernel<OT, D, 8>), grid, dim3(D), 0, stream, a, G);
  else if (a.nsplit <= 16)
    hipLaunchKernelGGL((attn_merge_kernel<OT, D, 16>), grid, dim3(D), 0, stream, a, G);
  else if (a.nsplit <= 32)
    hipLaunchKernelGGL((attn_merge_kernel<OT, D, 32>), grid, dim3(D), 0, stream, a, G);
  else if (a.nsplit <= 64)
    hipLaunchKernelGGL((attn_merge_kernel<OT, D, 64>), grid, dim3(D), 0, stream, a, G);
  else
    hipLaunchKernelGGL((attn_merge_wide_kernel<OT, D>), grid, dim3(D), 0, stream, a, G);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_p(int P, int tiles, const AttnArgs& a, int G, bool rope, int parts,
                           hipStream_t stream) {
  if (P == 16) return launch_tiles<T, D, 16>(tiles, a, G, rope, parts, stream);
  return launch_tiles<T, D, 32>(tiles, a, G, rope, parts, stream);
}

static hipError_t launch_parts(const LaunchKV& kv, const AttnArgs& a, bool rope, int parts,
                               hipStream_t stream) {
  const int tiles = tiles_for(kv, a.pps);
  if (kv.dtype == 2) {
    if (kv.D == 64) return launch_p<fp8_t, 64>(kv.P, tiles, a, kv.G, rope, parts, stream);
    return launch_p<fp8_t, 128>(kv.P, tiles, a, kv.G, rope, parts, stream);
  }
  if (kv.dtype == 0) {
    if (kv.D == 64) return launch_p<float, 64>(kv.P, tiles, a, kv.G, rope, parts, stream);
    return launch_p<float, 128>(kv.P, tiles, a, kv.G, rope, parts, stream);
  }
  if (kv.D == 64) return launch_p<bf16_t, 64>(kv.P, tiles, a, kv.G, rope, parts, stream);
  return launch_p<bf16_t, 128>(kv.P, tiles, a, kv.G, rope, parts, stream);
}

AttnArgs attn_args(const LaunchKV& kv, const RopeArgs& rope, const void* q, const int32_t* sel_idx,
                   const int32_t* sel_cnt, int k, float scale, int pps, void* out, float* lse,
                   void* ws) {
  AttnArgs a;
  a.k_pool = kv.k_pool;
  a.v_pool = kv.v_pool;
  a.page_table = kv.page_table;
  a.seq_lens = kv.seq_lens;
  a.q = q;
  a.sel_idx = sel_idx;
  a.sel_cnt = sel_cnt;
  a.Hkv = kv.Hkv;
  a.P = kv.P;
  a.log2P = kv.log2P;
  a.maxp = kv.maxp;
  a.maxn = kv.maxn;
  a.Npp = kv.Npp;
  a.k = k;
  a.pps = pps;
  a.nsplit = (k + pps - 1) / pps;
  a.nlists = kv.B * kv.Hkv;
  a.scale = scale;
  a.k_scale = kv.k_scale;
  a.v_scale = kv.v_scale;
  a.page_fill = kv.page_fill;
  a.rope = rope;
  a.part_acc = nullptr;
  a.part_ml = nullptr;
  if (a.nsplit > 1) {
    const size_t parts = (size_t)a.nlists * a.nsplit * kv.G;
    a.part_acc = (float*)ws;
    a.part_ml = (float4*)((char*)ws + align256(parts * kv.D * sizeof(float)));
  }
  a.out = out;
  a.lse = lse;
  a.scores = nullptr;
  a.sel_out = nullptr;
  a.cnt_out = nullptr;
  a.reuse = ReuseArgs{};
  return a;
}

hipError_t launch_attention(const LaunchKV& kv, const RopeArgs& rope, const void* q,
                            const int32_t* sel_idx, const int32_t* sel_cnt, int k, float scale,
                            int pages_per_split, void* out, float* lse, void* ws,
                            hipStream_t stream) {
  const int pps = attention_pages_per_split(kv, k, pages_per_split);
  const AttnArgs a = attn_args(kv, rope, q, sel_idx, sel_cnt, k, scale, pps, out, lse, ws);
  return launch_parts(kv, a, rope.page_row != nullptr, 3, stream);
}

hipError_t launch_merge(const LaunchKV& kv, const AttnArgs& a, hipStream_t stream) {
  return launch_parts(kv, a, false, 2, stream);
}

}  // namespace kvsel
