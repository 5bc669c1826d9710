// Segment-batch restore attention for gfx950.
//
// [CE] Appendix A.1.1 (Figure 10): a restore forward splits its queries at
// drop / reposition boundaries into segments; each segment applies standard
// causal attention over its own KV list, and all segments run in one batch.
// Here a segment reads one sequence of the cache (a position version made by
// akv_fork, or the original), whose last n entries are the segment's own
// tokens: query row i of an n-row segment attends to entries
// [0, len - n + i].
//
// The kernel is the decode kernel with the 16 MFMA columns holding
// (query token, head) pairs instead of padded heads: with GQA group G a
// column tile carries 16/G consecutive query tokens of one kv head, each
// column with its own causal limit.  Grid (query block, segment,
// layer x kv head); 8 waves split the block's causal page range and merge in
// LDS.  K goes from HBM straight into MFMA A-operand registers, V is staged
// per wave in LDS and read transposed for the PV MFMA.
#include "akv_internal.h"

#include <math.h>

namespace akv {

typedef __bf16 bf16x8s __attribute__((ext_vector_type(8)));
typedef short short4s __attribute__((ext_vector_type(4)));
typedef float floatx4s __attribute__((ext_vector_type(4)));

constexpr int kSegWaves = 8;

__device__ __forceinline__ bf16x8s seg_load8(const uint16_t *p) {
  return __builtin_bit_cast(bf16x8s, *reinterpret_cast<const uint4 *>(p));
}
__device__ __forceinline__ short seg_bf16(float x) { return __builtin_bit_cast(short, (__bf16)x); }

template <int D>
__global__ __launch_bounds__(kSegWaves * 64, 2) void segment_attn_kernel(
    Dev d, const uint16_t *__restrict__ q, const int32_t *__restrict__ seg_seq,
    const int32_t *__restrict__ seg_q_off, int max_q, int l0, int nL, int Hq,
    uint16_t *__restrict__ out) {
  constexpr int KC = D / 32, NT = D / 16, VC = D / 32, C8 = D / 8, VROW = D + 8;
  constexpr int kVBytes = kSegWaves * kPage * VROW * 2;
  constexpr int kOBytes = kSegWaves * 16 * D * 4;
  __shared__ __attribute__((aligned(16))) char s_raw[kVBytes > kOBytes ? kVBytes : kOBytes];
  __shared__ float s_m[kSegWaves][16], s_l[kSegWaves][16];
  auto s_v = reinterpret_cast<uint16_t (*)[kPage][VROW]>(s_raw);
  auto s_o = reinterpret_cast<float (*)[16][D]>(s_raw);

  const int G = Hq / d.H;
  const int TB = 16 / G;                       // query tokens per block
  const int sg = blockIdx.y;
  const int li = blockIdx.z / d.H, g = blockIdx.z - li * d.H, l = l0 + li;
  const int q0 = seg_q_off[sg];
  const int n = seg_q_off[sg + 1] - q0;
  const int i0 = blockIdx.x * TB;
  if (n < 0 || n > max_q) {
    if (threadIdx.x == 0 && blockIdx.x == 0 && blockIdx.z == 0)
      atomicCAS(&d.ctl[CTL_ERR], 0, (int)AKV_ERR_ARG);
    return;
  }
  if (i0 >= n) return;
  const int seq = seg_seq[sg];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int cl = lane & 15, kg = lane >> 4;
  const int tq = cl / G, hh = cl - tq * G;     // this lane's column: token tq, head hh
  const int len = (seq >= 0 && seq < d.B) ? d.lens[seq] : -1;
  const bool bad = len < n;
  if (bad && threadIdx.x == 0 && blockIdx.x == 0 && blockIdx.z == 0)
    atomicCAS(&d.ctl[CTL_ERR], 0, (int)AKV_ERR_ARG);
  const int i_col = i0 + tq;                   // row of this column inside the segment
  const bool col_ok = !bad && i_col < n;
  const int lim = col_ok ? len - n + i_col : -1;          // last visible entry
  const int i_last = min(i0 + TB, n) - 1;
  const int P = bad ? 0 : (len - n + i_last + 1 + kPage - 1) / kPage;

  bf16x8s qb[KC];
  {
    const uint16_t *qrow = q + (((size_t)(q0 + i_col) * nL + li) * Hq + (size_t)g * G + hh) * D;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      if (col_ok) qb[c] = seg_load8(qrow + 8 * kg + 32 * c);
      else qb[c] = __builtin_bit_cast(bf16x8s, make_uint4(0, 0, 0, 0));
    }
  }
  const float scale = 1.4426950408889634f / sqrtf((float)D);
  float m = -INFINITY, lsum = 0.f;
  floatx4s acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = floatx4s{0.f, 0.f, 0.f, 0.f};

  const int32_t *trow = d.table + (size_t)(bad ? 0 : seq) * d.maxpg;
  const PoolStrides ps = pool_strides(d.NB, d.H, D);
  const size_t head_base = (size_t)l * ps.layer + (size_t)g * ps.head;

  bf16x8s ka[KC];
  uint4 vv[VC];
  int p = wave;
  if (p < P) {
    const size_t off = head_base + (size_t)trow[p] * ps.page;
#pragma unroll
    for (int c = 0; c < KC; ++c) ka[c] = seg_load8(d.k + off + cl * D + 8 * kg + 32 * c);
#pragma unroll
    for (int c = 0; c < VC; ++c) vv[c] = *reinterpret_cast<const uint4 *>(d.v + off + 8 * (lane + 64 * c));
  }
  while (p < P) {
    const int pn = p + kSegWaves;
#pragma unroll
    for (int c = 0; c < VC; ++c) {
      const int ci = lane + 64 * c, row = ci / C8, col = (ci % C8) * 8;
      uint4 v = vv[c];
      if (p * kPage + row >= len) v = make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4 *>(&s_v[wave][row][col]) = v;
    }
    bf16x8s kan[KC];
    if (pn < P) {
      const size_t off = head_base + (size_t)trow[pn] * ps.page;
#pragma unroll
      for (int c = 0; c < KC; ++c) kan[c] = seg_load8(d.k + off + cl * D + 8 * kg + 32 * c);
#pragma unroll
      for (int c = 0; c < VC; ++c) vv[c] = *reinterpret_cast<const uint4 *>(d.v + off + 8 * (lane + 64 * c));
    }
    floatx4s sacc = floatx4s{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KC; ++c) sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[c], qb[c], sacc, 0, 0, 0);
    const int tok0 = p * kPage + 4 * kg;
    float sv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) sv[j] = (tok0 + j <= lim) ? sacc[j] * scale : -INFINITY;
    float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mnew = fmaxf(m, mx);
    // a column may see a page with nothing visible before any visible entry
    const float alpha = (m == -INFINITY) ? 0.f : exp2f(m - mnew);
    float pj[4], psum = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pj[j] = (sv[j] == -INFINITY) ? 0.f : exp2f(sv[j] - mnew);
      psum += pj[j];
    }
    lsum = lsum * alpha + psum;
    m = mnew;
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] *= alpha;
    const short4s pb = short4s{seg_bf16(pj[0]), seg_bf16(pj[1]), seg_bf16(pj[2]), seg_bf16(pj[3])};
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int col = 16 * t + cl;
      const short4s va = short4s{(short)s_v[wave][4 * kg + 0][col], (short)s_v[wave][4 * kg + 1][col],
                                 (short)s_v[wave][4 * kg + 2][col], (short)s_v[wave][4 * kg + 3][col]};
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, acc[t], 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < KC; ++c) ka[c] = kan[c];
    p = pn;
  }

  __syncthreads();
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (kg == 0) {
    s_m[wave][cl] = m;
    s_l[wave][cl] = lsum;
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) s_o[wave][cl][16 * t + 4 * kg + j] = acc[t][j];
  __syncthreads();
  for (int e = threadIdx.x; e < 16 * D; e += kSegWaves * 64) {
    const int c = e / D, dim = e - c * D;
    const int ti = i0 + c / G;
    if (ti >= n) continue;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kSegWaves; ++w) M = fmaxf(M, s_m[w][c]);
    float Lsum = 0.f, o = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kSegWaves; ++w) {
        const float f = s_m[w][c] == -INFINITY ? 0.f : exp2f(s_m[w][c] - M);
        Lsum += f * s_l[w][c];
        o += f * s_o[w][c][dim];
      }
    }
    const size_t orow = ((size_t)(q0 + ti) * nL + li) * Hq + (size_t)g * G + (c % G);
    out[orow * D + dim] = (uint16_t)seg_bf16(Lsum > 0.f ? o / Lsum : 0.f);
  }
}

hipError_t launch_segment_attention(const Dev &d, const uint16_t *q, const int32_t *seg_seq,
                                    const int32_t *seg_q_off, int n_seg, int max_q, int l0,
                                    int nL, int Hq, uint16_t *out, hipStream_t st) {
  const int G = Hq / d.H;
  const int TB = 16 / G;
  const dim3 grid((max_q + TB - 1) / TB, n_seg, nL * d.H), block(kSegWaves * 64);
  if (d.D == 128)
    hipLaunchKernelGGL(segment_attn_kernel<128>, grid, block, 0, st, d, q, seg_seq, seg_q_off,
                       max_q, l0, nL, Hq, out);
  else
    hipLaunchKernelGGL(segment_attn_kernel<64>, grid, block, 0, st, d, q, seg_seq, seg_q_off,
                       max_q, l0, nL, Hq, out);
  return hipGetLastError();
}

}  // namespace akv
