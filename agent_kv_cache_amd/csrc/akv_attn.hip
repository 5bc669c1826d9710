// Split-K GQA decode attention over the active KV, for gfx950.
//
// o = softmax(q K^T / sqrt(d)) V over the first active_len entries of each
// sequence (the active cache of [CE] sec. 3.1/3.3: dropped entries are no
// longer present after compaction, so only surviving KV is read).
//
// Grid: split x kv head x (sequence, layer), flattened with the split
// fastest; 8 waves per workgroup, wave w takes
// pages w, w+8, ... of the split.  Per 16-token page a wave
//   - loads K straight into MFMA A-operand registers (lane = token row,
//     16-B loads) and computes S^T[16 tok x 16 q-head] with
//     v_mfma_f32_16x16x32_bf16 (the GQA group is padded to 16 columns),
//   - does the online softmax in the MFMA output layout (4 tokens per lane,
//     row max/sum with two cross-lane xor shuffles),
//   - stages the V page in its own LDS slice and reads it transposed as the
//     A operand of v_mfma_f32_16x16x16_bf16, whose B operand P^T is exactly
//     the softmax output already held by the lane (no shuffles).
// The next page's K and V are loaded before the current one is consumed;
// K/V loads carry the nontemporal hint (each byte is read once).
// Waves merge through LDS; with several splits the partial (m, l, O) go to
// the workspace and a combine kernel merges them (log-sum-exp in base 2).
#include "akv_internal.h"

#include <math.h>

namespace akv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

#ifndef AKV_ATTN_WAVES
#define AKV_ATTN_WAVES 8       // waves per workgroup (pages interleaved across them)
#endif
#ifndef AKV_ATTN_MIN_WAVES
#define AKV_ATTN_MIN_WAVES 2   // waves per SIMD the register budget must allow
#endif
constexpr int kAttnWaves = AKV_ATTN_WAVES;

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t *p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(p));
}

#ifndef AKV_ATTN_NT
#define AKV_ATTN_NT 1          // nontemporal hint on the K/V page loads
#endif
typedef unsigned int u32x4a __attribute__((ext_vector_type(4)));
// K/V page loads: every KV byte is read once per decode step, so the loads
// carry the nontemporal hint (no cache retention); measured on the
// Llama-8B-shaped decode: 0.408 -> 0.361 ms (5.9 -> 6.6 TB/s).
__device__ __forceinline__ uint4 load_kv(const uint16_t *p) {
#if AKV_ATTN_NT
  const u32x4a v = __builtin_nontemporal_load(reinterpret_cast<const u32x4a *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
#else
  return *reinterpret_cast<const uint4 *>(p);
#endif
}

#ifndef AKV_ATTN_FAST_EXP
#define AKV_ATTN_FAST_EXP 0    // 1: softmax uses the bare v_exp_f32 (no denormal range reduction)
#endif
__device__ __forceinline__ float attn_exp2(float x) {
#if AKV_ATTN_FAST_EXP
  return __builtin_amdgcn_exp2f(x);
#else
  return exp2f(x);
#endif
}

__device__ __forceinline__ short f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(short, (__bf16)x);
}

template <int D>
__global__ __launch_bounds__(kAttnWaves * 64, AKV_ATTN_MIN_WAVES) void attn_kernel(
    Dev d, const uint16_t *__restrict__ q, const int32_t *__restrict__ active_len, int l0,
    int nL, int Hq, uint16_t *__restrict__ out, float *__restrict__ part, int nsplit,
    LayerOrder order) {
  constexpr int KC = D / 32;      // QK MFMA steps (K = 32 of d each)
  constexpr int NT = D / 16;      // PV output tiles of 16 dims
  constexpr int VC = D / 32;      // 16-B V chunks per lane per page
  constexpr int C8 = D / 8;       // 16-B chunks per row
  constexpr int VROW = D + 8;     // padded LDS row, elements
  // One LDS block serves two phases: per-wave V tiles in the page loop, then
  // the per-wave (m, l, O) of the final merge.
  constexpr int kVBytes = kAttnWaves * kPage * VROW * 2;
  constexpr int kOBytes = kAttnWaves * 16 * D * 4;
  __shared__ __attribute__((aligned(16))) char s_raw[kVBytes > kOBytes ? kVBytes : kOBytes];
  __shared__ float s_m[kAttnWaves][16], s_l[kAttnWaves][16];
  auto s_v = reinterpret_cast<uint16_t (*)[kPage][VROW]>(s_raw);
  auto s_o = reinterpret_cast<float (*)[16][D]>(s_raw);

  // one grid dimension, split fastest, then kv head, then (sequence, layer):
  // the dispatch order of a (split, head, sequence x layer) grid without its
  // 65535 limit on the last axis
  const int s = (int)(blockIdx.x % (unsigned)nsplit);
  const int gb = (int)(blockIdx.x / (unsigned)nsplit);
  const int g = gb % d.H, bl = gb / d.H;
  // With sliding-window layers the grid's layer axis runs over the ordered
  // layers (full attention first) with the sequences fastest, so the long
  // rows are dispatched first and spread over the CUs instead of pairing up
  // on the same CUs as full and window layers alternate.
  int b, li;
  if (order.n) {
    b = bl % d.B;
    li = order.idx[bl / d.B];
  } else {
    b = bl / nL;
    li = bl - b * nL;
  }
  const int l = l0 + li;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int hh = lane & 15, kg = lane >> 4;
  const int G = Hq / d.H;

  const int seqlen = d.lens[b];
  int len = active_len ? active_len[b] : seqlen;
  if (len < 0 || len > seqlen) {
    if (threadIdx.x == 0 && s == 0 && g == 0) atomicCAS(&d.ctl[CTL_ERR], 0, (int)AKV_ERR_ARG);
    len = len < 0 ? 0 : seqlen;
  }
  const int32_t *trow = d.table + (size_t)b * d.maxpg;
  // Sliding window: the query sits at next_pos and reads the entries whose
  // position is >= next_pos - W + 1; at most W - 1 entries qualify, so the
  // first of them is searched among the last W - 1.
  int f = 0;
  if (d.any_window) {
    const int W = d.window[l];
    if (W > 0) f = min(len, first_pos_at_least(d, trow, max(0, seqlen - W + 1), seqlen,
                                               d.next_pos[b] - W + 1));
  }
  const int P = (len + kPage - 1) / kPage;
  const int pstart = f / kPage;
  const int npg = f < len ? P - pstart : 0;
  const int chunk = (npg + nsplit - 1) / nsplit;
  const int p0 = pstart + s * chunk, p1 = min(pstart + npg, p0 + chunk);

  // Query rows as the B operand: column hh = query head g*G + hh.
  bf16x8 qb[KC];
  {
    const uint16_t *qrow = q + (((size_t)b * nL + li) * Hq + (size_t)g * G + hh) * D;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      if (hh < G) qb[c] = load_bf16x8(qrow + 8 * kg + 32 * c);
      else qb[c] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
    }
  }

  const float scale = 1.4426950408889634f / sqrtf((float)D);  // log2(e)/sqrt(d)
  float m = -INFINITY, lsum = 0.f;
  floatx4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};

  const PoolStrides ps = pool_strides(d.NB, d.H, D);
  const size_t head_base = (size_t)l * ps.layer + (size_t)g * ps.head;
  const size_t page_stride = ps.page;

  // Page p's K and V are in registers at the top of an iteration.  Its V goes
  // to LDS first, which frees the V registers for the next page's loads;
  // those and the next page's K loads stay in flight while page p is consumed.
  bf16x8 ka[KC];
  uint4 vv[VC];
  int p = p0 + wave;
  if (p < p1) {
    const size_t off = head_base + (size_t)trow[p] * page_stride;
#pragma unroll
    for (int c = 0; c < KC; ++c) ka[c] = __builtin_bit_cast(bf16x8, load_kv(d.k + off + hh * D + 8 * kg + 32 * c));
#pragma unroll
    for (int c = 0; c < VC; ++c) vv[c] = load_kv(d.v + off + 8 * (lane + 64 * c));
  }
  while (p < p1) {
    const int pn = p + kAttnWaves;
    // stage V (rows past the active length are zeroed: never multiply junk)
#pragma unroll
    for (int c = 0; c < VC; ++c) {
      const int ci = lane + 64 * c, row = ci / C8, col = (ci % C8) * 8;
      uint4 v = vv[c];
      if (p * kPage + row >= len) v = make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4 *>(&s_v[wave][row][col]) = v;
    }
    bf16x8 kan[KC];
    if (pn < p1) {
      const size_t off = head_base + (size_t)trow[pn] * page_stride;
#pragma unroll
      for (int c = 0; c < KC; ++c) kan[c] = __builtin_bit_cast(bf16x8, load_kv(d.k + off + hh * D + 8 * kg + 32 * c));
#pragma unroll
      for (int c = 0; c < VC; ++c) vv[c] = load_kv(d.v + off + 8 * (lane + 64 * c));
    }
    // S^T[token 4*kg + j][head hh]
    floatx4 sacc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KC; ++c) sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[c], qb[c], sacc, 0, 0, 0);
    const int tok0 = p * kPage + 4 * kg;
    float sv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) sv[j] = (tok0 + j < len && tok0 + j >= f) ? sacc[j] * scale : -INFINITY;
    float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mnew = fmaxf(m, mx);
    const float alpha = attn_exp2(m - mnew);
    float pj[4], ps = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pj[j] = attn_exp2(sv[j] - mnew);
      ps += pj[j];
    }
    lsum = lsum * alpha + ps;
    m = mnew;
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] *= alpha;
    const short4v pb = short4v{f32_to_bf16_bits(pj[0]), f32_to_bf16_bits(pj[1]),
                               f32_to_bf16_bits(pj[2]), f32_to_bf16_bits(pj[3])};
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int col = 16 * t + hh;
      const short4v va = short4v{(short)s_v[wave][4 * kg + 0][col], (short)s_v[wave][4 * kg + 1][col],
                                 (short)s_v[wave][4 * kg + 2][col], (short)s_v[wave][4 * kg + 3][col]};
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, acc[t], 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < KC; ++c) ka[c] = kan[c];
    p = pn;
  }

  // ---- merge the waves ----
  __syncthreads();  // all V tiles consumed before s_raw is reused
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (kg == 0) {
    s_m[wave][hh] = m;
    s_l[wave][hh] = lsum;
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) s_o[wave][hh][16 * t + 4 * kg + j] = acc[t][j];
  __syncthreads();
  const size_t row0 = ((size_t)b * nL + li) * Hq + (size_t)g * G;
  for (int e = threadIdx.x; e < G * D; e += kAttnWaves * 64) {
    const int h = e / D, dim = e - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, s_m[w][h]);
    float L = 0.f, o = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) {
        const float f = exp2f(s_m[w][h] - M);
        L += f * s_l[w][h];
        o += f * s_o[w][h][dim];
      }
    }
    if (nsplit == 1) {
      out[(row0 + h) * D + dim] = (uint16_t)f32_to_bf16_bits(L > 0.f ? o / L : 0.f);
    } else {
      float *pr = part + ((row0 + h) * nsplit + s) * (size_t)(D + 2);
      if (dim == 0) {
        pr[0] = M;
        pr[1] = L;
      }
      pr[2 + dim] = o;
    }
  }
}

// Merge split partials of one (sequence, layer, query head) row.  All split
// records of the row are loaded up front (independent loads in flight), in
// batches of AKV_COMBINE_UNROLL records (one dependent round trip per batch).
#ifndef AKV_COMBINE_UNROLL
#define AKV_COMBINE_UNROLL 16
#endif
template <int D>
__global__ __launch_bounds__(D) void combine_kernel(const float *__restrict__ part,
                                                    uint16_t *__restrict__ out, int nsplit) {
  constexpr int kMaxUnroll = AKV_COMBINE_UNROLL;
  const size_t row = blockIdx.x;
  const int dim = threadIdx.x;
  const float *pr = part + row * nsplit * (size_t)(D + 2);
  float M = -INFINITY, L = 0.f, o = 0.f;
  for (int s0 = 0; s0 < nsplit; s0 += kMaxUnroll) {
    const int n = min(kMaxUnroll, nsplit - s0);
    float ms[kMaxUnroll], ls[kMaxUnroll], os[kMaxUnroll];
    // unconditional loads (a record past the last split reads the last
    // one again and is then neutralised), so every load of the batch is
    // issued before the first wait
#pragma unroll
    for (int k = 0; k < kMaxUnroll; ++k) {
      const float *ps = pr + (size_t)(s0 + min(k, n - 1)) * (D + 2);
      ms[k] = ps[0];
      ls[k] = ps[1];
      os[k] = ps[2 + dim];
    }
#pragma unroll
    for (int k = 0; k < kMaxUnroll; ++k)
      if (k >= n) {
        ms[k] = -INFINITY;
        ls[k] = 0.f;
        os[k] = 0.f;
      }
    float Mn = M;
#pragma unroll
    for (int k = 0; k < kMaxUnroll; ++k) Mn = fmaxf(Mn, ms[k]);
    if (Mn != -INFINITY) {
      const float a = exp2f(M - Mn);   // M = -inf gives 0
      L *= a;
      o *= a;
#pragma unroll
      for (int k = 0; k < kMaxUnroll; ++k) {
        const float f = exp2f(ms[k] - Mn);
        L += f * ls[k];
        o += f * os[k];
      }
      M = Mn;
    }
  }
  out[row * D + dim] = (uint16_t)f32_to_bf16_bits(L > 0.f ? o / L : 0.f);
}

hipError_t launch_attention(const Dev &d, const uint16_t *q, const int32_t *active_len, int l0,
                            int nL, int Hq, uint16_t *out, float *part, int nsplit,
                            const LayerOrder &order, hipStream_t st) {
  const dim3 grid((unsigned)((long long)nsplit * d.H * d.B * nL)), block(kAttnWaves * 64);
  if (d.D == 128)
    hipLaunchKernelGGL(attn_kernel<128>, grid, block, 0, st, d, q, active_len, l0, nL, Hq, out,
                       part, nsplit, order);
  else
    hipLaunchKernelGGL(attn_kernel<64>, grid, block, 0, st, d, q, active_len, l0, nL, Hq, out,
                       part, nsplit, order);
  return hipGetLastError();
}

int attn_threads() { return kAttnWaves * 64; }

int attn_blocks_per_cu(int D) {
  int n = 0;
  const hipError_t e = (D == 128)
      ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_kernel<128>, kAttnWaves * 64, 0)
      : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_kernel<64>, kAttnWaves * 64, 0);
  return (e == hipSuccess && n > 0) ? n : 2;
}

hipError_t launch_combine(const float *part, uint16_t *out, int rows, int nsplit, int D,
                          hipStream_t st) {
  if (D == 128)
    hipLaunchKernelGGL(combine_kernel<128>, dim3(rows), dim3(128), 0, st, part, out, nsplit);
  else
    hipLaunchKernelGGL(combine_kernel<64>, dim3(rows), dim3(64), 0, st, part, out, nsplit);
  return hipGetLastError();
}

}  // namespace akv
