// Sparse paged decode attention (split-K over the selected pages) and the log-sum-exp merge.
//
// attn_split_kernel: one 256-thread block per (split, KV head, sequence). A split is pps
// consecutive entries of the selection list (pps * P rows); each of the 4 waves owns CPW chunks
// of RPW rows. All K and V loads of the block are issued before any arithmetic (16-byte
// coalesced slices, LPR lanes per row), so a block has its whole 2 * pps * P * D-element tile in
// flight at once. The whole GQA group (G query heads) is served from one read of K and V.
// Per wave: z = scale * q.k folded over the LPR lanes of a row, a wave-wide max, p = exp(z - m),
// l = sum p, acc = sum p * v folded over the row groups. The 4 waves are then merged through LDS
// and the block writes one (m, l, acc[D]) partial per query head -- or, with a single split,
// the normalized output directly.
//
// attn_merge_kernel: one block per (query head, sequence); thread d combines the partials of
// channel d: M = max m_s, out = sum_s e^(m_s - M) acc_s / sum_s e^(m_s - M) l_s.
#include <math.h>

#include "kvsel_device.h"
#include "kvsel_internal.h"

namespace kvsel {

template <typename T, int D, int G, int CPW>
__global__ __launch_bounds__(256) void attn_split_kernel(
    const T* __restrict__ k_pool, const T* __restrict__ v_pool,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ seq_lens,
    const T* __restrict__ q, const int32_t* __restrict__ sel_idx,
    const int32_t* __restrict__ sel_cnt, int Hkv, int P, int log2P, int maxp, int k, int pps,
    int nsplit, float scale, RopeArgs rope, float* __restrict__ part_acc,
    float2* __restrict__ part_ml, T* __restrict__ out, float* __restrict__ lse) {
  using M = row_map<T, D>;
  constexpr int VEC = M::VEC, LPR = M::LPR, RPW = M::RPW;
  const float NEG_INF = __int_as_float(0xff800000);

  const int split = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int rg = lane / LPR, c0 = (lane % LPR) * VEC;
  const size_t list = (size_t)b * Hkv + j;
  const int cnt = min(sel_cnt[list], k);
  const int L = seq_lens[b];
  const int Hq = Hkv * G;

  // ---- issue every K / V load of this wave first ----
  uint4 kraw[CPW], vraw[CPW];
  bool valid[CPW];
  int rrow[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int r0 = (w * CPW + i) * RPW;  // first row of the chunk (wave-uniform)
    const int sp = split * pps + (r0 >> log2P);
    const int s = (r0 & (P - 1)) + rg;
    bool ok = false;
    size_t off = 0;
    rrow[i] = -1;
    if (sp < cnt) {
      const int n = sel_idx[list * k + sp];
      const int p = n >= 0 && n < maxp ? page_table[(size_t)b * maxp + n] : 0;
      ok = n >= 0 && n < maxp && n * P + s < L;
      off = (((size_t)p * Hkv + j) * P + s) * D + c0;
      if (rope.page_row) {
        const int pr = rope.page_row[p];
        rrow[i] = pr < 0 ? -1 : pr + rope.row_step * s;
      }
    }
    kraw[i] = ok ? load16(k_pool + off) : make_uint4(0, 0, 0, 0);
    vraw[i] = ok ? load16(v_pool + off) : make_uint4(0, 0, 0, 0);
    valid[i] = ok;
  }

  float qf[G][VEC];
#pragma unroll
  for (int g = 0; g < G; ++g) unpack<T>(load16(q + ((size_t)b * Hq + j * G + g) * D + c0), qf[g]);

  // ---- scores of this wave's rows ----
  float z[CPW][G];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    float kf[VEC];
    unpack<T>(kraw[i], kf);
    if (rope.page_row) rope_rotate_slice<T, D>(kf, c0, rrow[i], rope.cos, rope.sin);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) s = fmaf(qf[g][e], kf[e], s);
#pragma unroll
      for (int m = 1; m < LPR; m <<= 1) s += __shfl_xor(s, m);
      z[i][g] = valid[i] ? s * scale : NEG_INF;
    }
  }
  float mx[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float m = z[0][g];
#pragma unroll
    for (int i = 1; i < CPW; ++i) m = fmaxf(m, z[i][g]);
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
    mx[g] = m;
  }
  float l[G], acc[G][VEC];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    l[g] = 0.0f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[g][e] = 0.0f;
  }
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    float vf[VEC];
    unpack<T>(vraw[i], vf);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float pz = valid[i] ? __expf(z[i][g] - mx[g]) : 0.0f;
      l[g] += pz;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[g][e] = fmaf(pz, vf[e], acc[g][e]);
    }
  }
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      l[g] += __shfl_xor(l[g], o);
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[g][e] += __shfl_xor(acc[g][e], o);
    }
  }

  // ---- merge the 4 waves ----
  __shared__ float s_m[4][G], s_l[4][G];
  __shared__ float s_acc[4][G][D];
  if (rg == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < VEC; ++e) s_acc[w][g][c0 + e] = acc[g][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      s_m[w][g] = mx[g];
      s_l[w][g] = l[g];
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += 256) {
    const int g = idx / D, d = idx % D;
    float Mx = s_m[0][g];
#pragma unroll
    for (int v = 1; v < 4; ++v) Mx = fmaxf(Mx, s_m[v][g]);
    float Ls = 0.0f, A = 0.0f;
    if (Mx != NEG_INF) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (s_m[v][g] != NEG_INF) {
          const float f = __expf(s_m[v][g] - Mx);
          Ls = fmaf(s_l[v][g], f, Ls);
          A = fmaf(s_acc[v][g][d], f, A);
        }
      }
    }
    if (nsplit == 1) {
      const size_t o = ((size_t)b * Hq + j * G + g) * D + d;
      store_elem<T>(out, o, Mx == NEG_INF ? 0.0f : A / Ls);
      if (d == 0 && lse) lse[(size_t)b * Hq + j * G + g] = Mx == NEG_INF ? NEG_INF : Mx + logf(Ls);
    } else {
      const size_t ps = (list * nsplit + split) * G + g;
      part_acc[ps * D + d] = A;
      if (d == 0) part_ml[ps] = make_float2(Mx, Ls);
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(128) void attn_merge_kernel(const float* __restrict__ part_acc,
                                                         const float2* __restrict__ part_ml,
                                                         int Hkv, int G, int nsplit,
                                                         T* __restrict__ out, float* __restrict__ lse) {
  const float NEG_INF = __int_as_float(0xff800000);
  const int h = blockIdx.x, b = blockIdx.y;
  const int j = h / G, g = h % G;
  const size_t list = (size_t)b * Hkv + j;
  const int Hq = Hkv * G;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float Mx = NEG_INF;
    for (int s = 0; s < nsplit; ++s) Mx = fmaxf(Mx, part_ml[(list * nsplit + s) * G + g].x);
    const size_t o = ((size_t)b * Hq + h) * D + d;
    if (Mx == NEG_INF) {
      store_elem<T>(out, o, 0.0f);
      if (d == 0 && lse) lse[(size_t)b * Hq + h] = NEG_INF;
      continue;
    }
    float Ls = 0.0f, A = 0.0f;
    for (int s = 0; s < nsplit; ++s) {
      const size_t ps = (list * nsplit + s) * G + g;
      const float2 ml = part_ml[ps];
      if (ml.x != NEG_INF) {
        const float f = __expf(ml.x - Mx);
        Ls = fmaf(ml.y, f, Ls);
        A = fmaf(part_acc[ps * D + d], f, A);
      }
    }
    store_elem<T>(out, o, A / Ls);
    if (d == 0 && lse) lse[(size_t)b * Hq + h] = Mx + logf(Ls);
  }
}

// ---- host side ----

static int rows_per_wave_load(const LaunchKV& kv) {
  const int vec = kv.dtype == 0 ? 4 : 8;
  return 64 / (kv.D / vec);
}

// Chunks per wave for a split of pps pages, or 0 when that split size has no kernel.
static int chunks_per_wave(const LaunchKV& kv, int pps) {
  const int rows = pps * kv.P;
  const int per = 4 * rows_per_wave_load(kv);
  if (rows % per) return 0;
  const int cpw = rows / per;
  return (cpw == 1 || cpw == 2 || cpw == 4 || cpw == 8) ? cpw : 0;
}

int attention_pages_per_split(const LaunchKV& kv, int k, int requested) {
  (void)k;
  int want = requested > 0 ? requested : 2;
  // largest supported split not above the request, else the smallest supported one
  for (int p = want; p >= 1; --p)
    if (chunks_per_wave(kv, p)) return p;
  for (int p = want + 1; p <= 64; ++p)
    if (chunks_per_wave(kv, p)) return p;
  return 0;
}

size_t attention_workspace(const LaunchKV& kv, int k, int pages_per_split) {
  const int pps = attention_pages_per_split(kv, k, pages_per_split);
  if (pps <= 0) return 0;
  const size_t nsplit = (size_t)((k + pps - 1) / pps);
  if (nsplit <= 1) return 0;
  const size_t parts = (size_t)kv.B * kv.Hkv * nsplit * kv.G;
  const size_t acc_bytes = parts * kv.D * sizeof(float);
  return ((acc_bytes + 255) & ~(size_t)255) + parts * sizeof(float2);
}

template <typename T, int D, int G, int CPW>
static void launch_split(const LaunchKV& kv, const RopeArgs& rope, const void* q,
                         const int32_t* sel_idx, const int32_t* sel_cnt, int k, float scale,
                         int pps, int nsplit, float* part_acc, float2* part_ml, void* out,
                         float* lse, hipStream_t stream) {
  hipLaunchKernelGGL((attn_split_kernel<T, D, G, CPW>),
                     dim3((unsigned)nsplit, (unsigned)kv.Hkv, (unsigned)kv.B), dim3(256), 0, stream,
                     (const T*)kv.k_pool, (const T*)kv.v_pool, kv.page_table, kv.seq_lens,
                     (const T*)q, sel_idx, sel_cnt, kv.Hkv, kv.P, kv.log2P, kv.maxp, k, pps, nsplit,
                     scale, rope, part_acc, part_ml, (T*)out, lse);
}

template <typename T, int D, int G>
static void launch_split_cpw(int cpw, const LaunchKV& kv, const RopeArgs& rope, const void* q,
                             const int32_t* sel_idx, const int32_t* sel_cnt, int k, float scale,
                             int pps, int nsplit, float* part_acc, float2* part_ml, void* out,
                             float* lse, hipStream_t stream) {
  switch (cpw) {
    case 1: launch_split<T, D, G, 1>(kv, rope, q, sel_idx, sel_cnt, k, scale, pps, nsplit, part_acc, part_ml, out, lse, stream); break;
    case 2: launch_split<T, D, G, 2>(kv, rope, q, sel_idx, sel_cnt, k, scale, pps, nsplit, part_acc, part_ml, out, lse, stream); break;
    case 4: launch_split<T, D, G, 4>(kv, rope, q, sel_idx, sel_cnt, k, scale, pps, nsplit, part_acc, part_ml, out, lse, stream); break;
    default: launch_split<T, D, G, 8>(kv, rope, q, sel_idx, sel_cnt, k, scale, pps, nsplit, part_acc, part_ml, out, lse, stream); break;
  }
}

template <typename T, int D>
static hipError_t launch_attention_t(const LaunchKV& kv, const RopeArgs& rope, const void* q,
                                     const int32_t* sel_idx, const int32_t* sel_cnt, int k,
                                     float scale, int pps, void* out, float* lse, void* ws,
                                     hipStream_t stream) {
  const int nsplit = (k + pps - 1) / pps;
  const int cpw = chunks_per_wave(kv, pps);
  float* part_acc = nullptr;
  float2* part_ml = nullptr;
  if (nsplit > 1) {
    const size_t parts = (size_t)kv.B * kv.Hkv * nsplit * kv.G;
    part_acc = (float*)ws;
    part_ml = (float2*)((char*)ws + (((parts * kv.D * sizeof(float)) + 255) & ~(size_t)255));
  }
  switch (kv.G) {
    case 1: launch_split_cpw<T, D, 1>(cpw, kv, rope, q, sel_idx, sel_cnt, k, scale, pps, nsplit, part_acc, part_ml, out, lse, stream); break;
    case 2: launch_split_cpw<T, D, 2>(cpw, kv, rope, q, sel_idx, sel_cnt, k, scale, pps, nsplit, part_acc, part_ml, out, lse, stream); break;
    case 4: launch_split_cpw<T, D, 4>(cpw, kv, rope, q, sel_idx, sel_cnt, k, scale, pps, nsplit, part_acc, part_ml, out, lse, stream); break;
    default: launch_split_cpw<T, D, 8>(cpw, kv, rope, q, sel_idx, sel_cnt, k, scale, pps, nsplit, part_acc, part_ml, out, lse, stream); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  hipLaunchKernelGGL((attn_merge_kernel<T, D>), dim3((unsigned)kv.Hq, (unsigned)kv.B),
                     dim3(D < 128 ? D : 128), 0, stream, part_acc, part_ml, kv.Hkv, kv.G, nsplit,
                     (T*)out, lse);
  return hipGetLastError();
}

hipError_t launch_attention(const LaunchKV& kv, const RopeArgs& rope, const void* q,
                            const int32_t* sel_idx, const int32_t* sel_cnt, int k, float scale,
                            int pages_per_split, void* out, float* lse, void* ws,
                            hipStream_t stream) {
  const int pps = attention_pages_per_split(kv, k, pages_per_split);
  if (kv.dtype == 0) {
    if (kv.D == 64)
      return launch_attention_t<float, 64>(kv, rope, q, sel_idx, sel_cnt, k, scale, pps, out, lse, ws, stream);
    return launch_attention_t<float, 128>(kv, rope, q, sel_idx, sel_cnt, k, scale, pps, out, lse, ws, stream);
  }
  if (kv.D == 64)
    return launch_attention_t<bf16_t, 64>(kv, rope, q, sel_idx, sel_cnt, k, scale, pps, out, lse, ws, stream);
  return launch_attention_t<bf16_t, 128>(kv, rope, q, sel_idx, sel_cnt, k, scale, pps, out, lse, ws, stream);
}

}  // namespace kvsel
