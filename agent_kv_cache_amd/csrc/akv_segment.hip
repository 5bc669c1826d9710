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

#include <limits.h>
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
// 2^x as the single hardware instruction (no denormal range reduction:
// results below 2^-126 flush to zero, which softmax weights can afford).
__device__ __forceinline__ float seg_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

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
  const bool col_ok = !bad && tq < TB && i_col < n;
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

  // Sliding window: a row at position p_i reads entries with position >=
  // p_i - W + 1 (at most W entries up to itself).  Pages before the first
  // row's first visible entry are skipped; the rest are masked by position.
  const int W = (d.any_window && !bad) ? d.window[l] : 0;
  int wlo = INT_MIN, pstart = 0;
  if (W > 0) {
    if (col_ok) wlo = entry_pos(d, trow, lim) - W + 1;
    const int me0 = len - n + i0;
    pstart = first_pos_at_least(d, trow, max(0, me0 - W + 1), me0 + 1,
                                entry_pos(d, trow, me0) - W + 1) / kPage;
  }

  bf16x8s ka[KC];
  uint4 vv[VC];
  int4 pp = make_int4(0, 0, 0, 0);                 // positions of this lane's 4 entries
  int p = pstart + wave;
  if (p < P) {
    const size_t off = head_base + (size_t)trow[p] * ps.page;
#pragma unroll
    for (int c = 0; c < KC; ++c) ka[c] = seg_load8(d.k + off + cl * D + 8 * kg + 32 * c);
#pragma unroll
    for (int c = 0; c < VC; ++c) vv[c] = *reinterpret_cast<const uint4 *>(d.v + off + 8 * (lane + 64 * c));
    if (W > 0) pp = *reinterpret_cast<const int4 *>(d.pos + (size_t)trow[p] * kPage + 4 * kg);
  }
  while (p < P) {
    const int pn = p + kSegWaves;
    const int4 pcur = pp;
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
      if (W > 0) pp = *reinterpret_cast<const int4 *>(d.pos + (size_t)trow[pn] * kPage + 4 * kg);
    }
    floatx4s sacc = floatx4s{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KC; ++c) sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[c], qb[c], sacc, 0, 0, 0);
    const int tok0 = p * kPage + 4 * kg;
    const int pj4[4] = {pcur.x, pcur.y, pcur.z, pcur.w};
    float sv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      sv[j] = (tok0 + j <= lim && (W == 0 || pj4[j] >= wlo)) ? sacc[j] * scale : -INFINITY;
    float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mnew = fmaxf(m, mx);
    // a column may see a page with nothing visible before any visible entry
    const float alpha = (m == -INFINITY) ? 0.f : seg_exp2(m - mnew);
    float pj[4], psum = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pj[j] = (sv[j] == -INFINITY) ? 0.f : seg_exp2(sv[j] - mnew);
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
    if (c / G >= TB || ti >= n) continue;      // columns past 16/G tokens belong to no row
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kSegWaves; ++w) M = fmaxf(M, s_m[w][c]);
    float Lsum = 0.f, o = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kSegWaves; ++w) {
        const float f = s_m[w][c] == -INFINITY ? 0.f : seg_exp2(s_m[w][c] - M);
        Lsum += f * s_l[w][c];
        o += f * s_o[w][c][dim];
      }
    }
    const size_t orow = ((size_t)(q0 + ti) * nL + li) * Hq + (size_t)g * G + (c % G);
    out[orow * D + dim] = (uint16_t)seg_bf16(Lsum > 0.f ? o / Lsum : 0.f);
  }
}

// ---------------------------------------------------------------------------
// Long segments: a prefill-shaped kernel.  A workgroup owns 256 columns
// (256/G query tokens x G heads of one kv head); each of its 8 waves owns 32
// of them (two MFMA column tiles) and keeps their Q fragments, exponent
// references, weight sums and O^T accumulators in registers.  The workgroup sweeps the
// causal KV range in 64-token tiles staged in LDS (K as rows, V transposed)
// (K double-buffered, V triple-buffered): the next tile's global loads are in
// flight while the current one is multiplied, so every KV byte is fetched
// once per workgroup and reused by 256 columns.
//   S^T tile (16 tokens x 16 columns) = K (16 x 32 dims) * Q^T, 16x16x32 MFMA.
//   O^T (16 dims x 16 columns) += V^T (16 dims x 32 tokens) * P^T: the 32
//   tokens of one MFMA step are ordered so that a lane's 8 k-values are the
//   4 + 4 probabilities it already holds from two S^T tiles.
//   Each column's weight sum is one more MFMA (a ones operand times P^T).
// Per tile a wave's MFMA time and its softmax VALU time (half of it the
// quarter-rate exponentials) are about equal, and a wave's QK -> softmax ->
// PV chain is serial; the waves of a SIMD also run in step (one barrier per
// tile).  So a tile's PV product is taken one iteration late, in the same
// basic block as the next tile's exponentials: the two are independent, and
// the matrix core multiplies while the VALU exponentiates.  The accumulation
// order is unchanged (a moved reference scales the sum that includes the
// previous tile, then the next tile is added).  The loop keeps other VALU
// work small (per-thread load offsets fixed before the sweep, zeroing only
// on the tile where the sequence ends, a reference that moves lazily,
// cross-row maxima with the row-swap instructions).
// ---------------------------------------------------------------------------
#ifndef AKV_FA_VPAD
#define AKV_FA_VPAD 4      // halfwords of padding per transposed-V row in LDS
#endif
#ifndef AKV_FA_KPAD
#define AKV_FA_KPAD 8      // halfwords of padding per K row in LDS (keeps 16-B alignment)
#endif
#ifndef AKV_FA_WAVES
#define AKV_FA_WAVES 8     // waves per workgroup (16 * AKV_FA_CT columns each)
#endif
#ifndef AKV_FA_MIN_WAVES
#define AKV_FA_MIN_WAVES 1 // waves per SIMD the register budget must allow
#endif
#ifndef AKV_FA_CT
#define AKV_FA_CT 2        // 16-column MFMA tiles per wave
#endif
constexpr int kFaWaves = AKV_FA_WAVES, kFaCT = AKV_FA_CT, kFaKT = 64,
              kFaCols = 16 * kFaCT * kFaWaves;
#ifndef AKV_FA_TAU
#define AKV_FA_TAU 8.0f    // log2 of the largest weight allowed before a column's reference moves
#endif
#ifndef AKV_FA_XCD
#define AKV_FA_XCD 1       // XCD-aware block order (see fa_block)
#endif
constexpr int kXcds = 8;   // MI355X: 8 accelerator dies, each with its own L2

// Block order.  The hardware hands workgroup L (linear id) to die L mod 8,
// in order of L; every query block of one (segment, layer, kv head) group
// sweeps the same K/V pages from the start.  Consecutive ids are therefore
// remapped so that die k runs whole groups one after another (groups k,
// k + 8, k + 16, ...; all query blocks of a group in a row): the ~32 blocks
// a die runs at once share one group's K/V tiles through that die's L2,
// instead of every die fetching every group's pages.  Within a group the
// query blocks run longest first (later rows see more entries), which
// trims the end of the launch.  Identity when the group count is not a
// multiple of the die count.
__device__ __forceinline__ void fa_block(int &bx, int &by, int &bz) {
  bx = blockIdx.x;
  by = blockIdx.y;
  bz = blockIdx.z;
  const int X = gridDim.x, Y = gridDim.y;
  const long long groups = (long long)Y * gridDim.z;
  if (!AKV_FA_XCD || groups % kXcds != 0) return;
  const long long L = bx + (long long)X * (by + (long long)Y * bz);
  const long long s = L / kXcds;                 // position in the die's order
  const long long gg = (s / X) * kXcds + L % kXcds;
  bx = X - 1 - (int)(s % X);   // a group's longest (latest) query blocks first
  by = (int)(gg % Y);
  bz = (int)(gg / Y);
}

// Maximum over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four 16-lane rows of a
// wave, which hold the same MFMA column), with the gfx950 row-swap
// instructions; every lane gets the same value.
__device__ __forceinline__ float fa_rows_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

template <int D>
__global__ __launch_bounds__(kFaWaves * 64, AKV_FA_MIN_WAVES) void segment_fa_kernel(
    Dev d, const uint16_t *__restrict__ q, const int32_t *__restrict__ seg_seq,
    const int32_t *__restrict__ seg_q_off, int max_q, int l0, int nL, int Hq,
    uint16_t *__restrict__ out) {
  constexpr int KC = D / 32, NT = D / 16, C8 = D / 8;
  constexpr int KROW = D + AKV_FA_KPAD, VROW = kFaKT + AKV_FA_VPAD;
  constexpr int NTH = kFaWaves * 64;
  constexpr int KPT = kFaKT * C8 / NTH;                  // K chunks per thread
  constexpr int VPAIRS = (kFaKT / 2) * C8;               // V token-pair chunks per tile
  constexpr int VPT = (VPAIRS + NTH - 1) / NTH;
  static_assert(KPT * NTH == kFaKT * C8, "K tile must split evenly");
  __shared__ __attribute__((aligned(16))) uint16_t s_k[2][kFaKT][KROW];
  __shared__ __attribute__((aligned(16))) uint16_t s_vt[3][D][VROW];
  __shared__ __attribute__((aligned(16))) int32_t s_pos[2][kFaKT];   // sliding-window layers only

  const int G = Hq / d.H;
  const int TBW = kFaCols / G;                            // query tokens per workgroup
  int bx, by, bz;
  fa_block(bx, by, bz);
  const int sg = by;
  const int li = bz / d.H, g = bz - li * d.H, l = l0 + li;
  const int q0 = seg_q_off[sg];
  const int n = seg_q_off[sg + 1] - q0;
  if (n < 0 || n > max_q) {
    if (threadIdx.x == 0 && bx == 0 && bz == 0)
      atomicCAS(&d.ctl[CTL_ERR], 0, (int)AKV_ERR_ARG);
    return;
  }
  const int i0 = bx * TBW;
  if (i0 >= n) return;
  const int seq = seg_seq[sg];
  const int len = (seq >= 0 && seq < d.B) ? d.lens[seq] : -1;
  const bool bad = len < n;
  if (bad && threadIdx.x == 0 && bx == 0 && bz == 0)
    atomicCAS(&d.ctl[CTL_ERR], 0, (int)AKV_ERR_ARG);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int cl = lane & 15, kg = lane >> 4;

  // this lane's column in each of the wave's column tiles
  int lim[kFaCT];
  bool rok[kFaCT], cok[kFaCT];   // the column is a row of the segment / and the segment is valid
  size_t qrow[kFaCT];
#pragma unroll
  for (int ct = 0; ct < kFaCT; ++ct) {
    const int c = 16 * kFaCT * wave + 16 * ct + cl;
    const int tq = c / G, hh = c - tq * G, i = i0 + tq;
    rok[ct] = tq < TBW && i < n;
    cok[ct] = !bad && rok[ct];
    lim[ct] = cok[ct] ? len - n + i : -1;
    qrow[ct] = ((size_t)(q0 + (rok[ct] ? i : 0)) * nL + li) * Hq + (size_t)g * G + hh;
  }
  // last entry any valid column of this wave sees, and the first entry some
  // valid column cannot see (tiles wholly before it need no causal mask)
  int wave_lim = -1, wave_lo = -1;
  {
    const int tlo = (16 * kFaCT * wave) / G, thi = min((16 * kFaCT * wave + 16 * kFaCT - 1) / G, TBW - 1);
    if (!bad && tlo < TBW && i0 + tlo < n) {
      wave_lim = len - n + min(i0 + thi, n - 1);
      wave_lo = len - n + i0 + tlo;
    }
  }
  const int last = bad ? -1 : len - n + min(i0 + TBW, n) - 1;
  const int ntile = (last + kFaKT) / kFaKT;
  const int32_t *trow = d.table + (size_t)(bad ? 0 : seq) * d.maxpg;

  // Sliding window: a row at position p_i reads the entries with position
  // >= p_i - W + 1.  The sweep starts at the tile of the first row's first
  // visible entry; entries are masked by position (kept in LDS per tile).
  const int W = (d.any_window && !bad) ? d.window[l] : 0;
  int wlo[kFaCT];
#pragma unroll
  for (int ct = 0; ct < kFaCT; ++ct) wlo[ct] = INT_MIN;
  int t0 = 0;
  if (W > 0) {
#pragma unroll
    for (int ct = 0; ct < kFaCT; ++ct)
      if (cok[ct]) wlo[ct] = entry_pos(d, trow, lim[ct]) - W + 1;
    const int me0 = len - n + i0;
    t0 = first_pos_at_least(d, trow, max(0, me0 - W + 1), me0 + 1,
                            entry_pos(d, trow, me0) - W + 1) / kFaKT;
  }

  bf16x8s qf[kFaCT][KC];
#pragma unroll
  for (int ct = 0; ct < kFaCT; ++ct)
#pragma unroll
    for (int c = 0; c < KC; ++c)
      qf[ct][c] = cok[ct] ? seg_load8(q + qrow[ct] * D + 8 * kg + 32 * c)
                          : __builtin_bit_cast(bf16x8s, make_uint4(0, 0, 0, 0));

  const float scale = 1.4426950408889634f / sqrtf((float)D);
  // Per column: the exponent reference in log2 units, -inf until a score is
  // visible.  Weights are p = 2^(s*scale - ref).  The reference moves to the
  // running maximum only when a score exceeds it by more than 2^AKV_FA_TAU,
  // so weights lie in [0, 2^AKV_FA_TAU] and the accumulators are rescaled on
  // few tiles; the final division by the sum of the same bf16 weights
  // cancels the reference.
  // nref = -ref (0 while ref = -inf); thr = the exponent above which the
  // reference moves (-inf while nothing is visible, then AKV_FA_TAU)
  float nref[kFaCT], thr[kFaCT];
  floatx4s acc[kFaCT][NT], lacc[kFaCT];
#pragma unroll
  for (int ct = 0; ct < kFaCT; ++ct) {
    nref[ct] = 0.f;
    thr[ct] = -INFINITY;
    lacc[ct] = floatx4s{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[ct][t] = floatx4s{0.f, 0.f, 0.f, 0.f};
  }
  // 1.0 in every k-slot: ones x P^T gives each column's weight sum on the
  // matrix core (every row of lacc holds it)
  const bf16x8s ones = __builtin_bit_cast(bf16x8s, make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));

  const PoolStrides ps = pool_strides(d.NB, d.H, D);
  const uint16_t *kb = d.k + (size_t)l * ps.layer + (size_t)g * ps.head;
  const uint16_t *vb = d.v + (size_t)l * ps.layer + (size_t)g * ps.head;
  const uint32_t pstride = (uint32_t)ps.page;           // elements per page

  // What each thread loads is fixed: K chunk r is 16-B chunk ck of tile row
  // tk[r]; V pair r is chunk vc[r] of rows 2 va[r] and 2 va[r] + 1.  Tiles
  // start on page boundaries, so tile row x lies in the tile's page x / 16,
  // at row x % 16 of that page: the in-page offsets are set once here and
  // each load adds one page base (a 32 x 32 -> 64-bit multiply-add).
  int tk[KPT], va[VPT], vc[VPT];
  bool von[VPT];
  const int ck = tid % C8;
  const uint16_t *kbt[KPT], *vbt[VPT];
#pragma unroll
  for (int r = 0; r < KPT; ++r) {
    tk[r] = (tid + NTH * r) / C8;
    kbt[r] = kb + (tk[r] & 15) * D + 8 * ck;
  }
#pragma unroll
  for (int r = 0; r < VPT; ++r) {
    const int idx = tid + NTH * r;
    von[r] = idx < VPAIRS;
    va[r] = von[r] ? (idx & 31) : 0;
    vc[r] = von[r] ? (idx >> 5) : 0;
    vbt[r] = vb + ((2 * va[r]) & 15) * D + 8 * vc[r];
  }
  const int lastp = (max(len, 1) - 1) >> 4;            // last page of the sequence

  // Page ids of the tile fetched next are loaded one tile ahead, so a
  // tile's K/V loads never wait on a table lookup.  Rows past the end of the
  // sequence read a row of its last page (always a valid address) and are
  // zeroed by value, so every load is unconditional.  Only called when
  // len >= 1.
  int pk[KPT], pv[VPT], pq = 0;
  auto pidx = [&](int t) {
    const int p0 = t * (kFaKT / kPage);
    if (W > 0 && tid < kFaKT) pq = trow[min(t * kFaKT + tid, len - 1) >> 4];
#pragma unroll
    for (int r = 0; r < KPT; ++r) pk[r] = trow[min(p0 + (tk[r] >> 4), lastp)];
#pragma unroll
    for (int r = 0; r < VPT; ++r) pv[r] = trow[min(p0 + ((2 * va[r]) >> 4), lastp)];
  };
  uint4 rk[KPT], rv[2 * VPT];
  int rpos = 0;
  auto gload = [&](int t) {
    if (W > 0 && tid < kFaKT) rpos = d.pos[(size_t)pq * kPage + (min(t * kFaKT + tid, len - 1) & 15)];
#pragma unroll
    for (int r = 0; r < KPT; ++r)
      rk[r] = *reinterpret_cast<const uint4 *>(kbt[r] + (uint64_t)(uint32_t)pk[r] * pstride);
#pragma unroll
    for (int r = 0; r < VPT; ++r) {
      // rows 2a and 2a + 1 share a page
      const uint16_t *pg = vbt[r] + (uint64_t)(uint32_t)pv[r] * pstride;
      rv[2 * r] = *reinterpret_cast<const uint4 *>(pg);
      rv[2 * r + 1] = *reinterpret_cast<const uint4 *>(pg + D);
    }
  };
  // registers -> LDS (V transposed); rows past the end of the sequence
  // become zeros here, which only the tile holding its end needs
  auto lstore = [&](int t, int buf, int vbuf) {
    const int T0 = t * kFaKT;
    if (W > 0 && tid < kFaKT) s_pos[buf][tid] = rpos;
    if (T0 + kFaKT > len) {
#pragma unroll
      for (int r = 0; r < KPT; ++r)
        if (T0 + tk[r] >= len) rk[r] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int r = 0; r < VPT; ++r) {
        const int e = T0 + 2 * va[r];
        if (e >= len) rv[2 * r] = make_uint4(0u, 0u, 0u, 0u);
        if (e + 1 >= len) rv[2 * r + 1] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int r = 0; r < KPT; ++r) *reinterpret_cast<uint4 *>(&s_k[buf][tk[r]][8 * ck]) = rk[r];
#pragma unroll
    for (int r = 0; r < VPT; ++r) {
      if (von[r]) {
        const int a = va[r], ch = vc[r];
        const uint4 v0 = rv[2 * r], v1 = rv[2 * r + 1];
        const uint32_t x0[4] = {v0.x, v0.y, v0.z, v0.w}, x1[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          // dims 8ch+2w (low halves) and 8ch+2w+1 (high halves) of rows 2a, 2a+1
          *reinterpret_cast<uint32_t *>(&s_vt[vbuf][8 * ch + 2 * w][2 * a]) =
              __builtin_amdgcn_perm(x1[w], x0[w], 0x05040100u);
          *reinterpret_cast<uint32_t *>(&s_vt[vbuf][8 * ch + 2 * w + 1][2 * a]) =
              __builtin_amdgcn_perm(x1[w], x0[w], 0x07060302u);
        }
      }
    }
  };

  if (t0 < ntile) {
    pidx(t0);
    gload(t0);
    if (t0 + 1 < ntile) pidx(t0 + 1);
    lstore(t0, 0, 0);
  }
  // V buffer 2 holds zeros for the first tile's (empty) pending product
  for (int e = tid; e < D * VROW / 8; e += NTH)
    reinterpret_cast<uint4 *>(&s_vt[2][0][0])[e] = make_uint4(0u, 0u, 0u, 0u);
  // Q and the first tile are in registers / LDS before the loop: no wait on
  // the loop's own prefetches inside it
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // O^T += V^T P^T and the weight sums for one tile's probabilities
  auto pv_tile = [&](const bf16x8s (&p)[kFaCT][2], int vbuf) {
#pragma unroll
    for (int ct = 0; ct < kFaCT; ++ct)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
        lacc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, p[ct][kc], lacc[ct], 0, 0, 0);
#pragma unroll
    for (int dt = 0; dt < NT; ++dt)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const uint2 lo = *reinterpret_cast<const uint2 *>(&s_vt[vbuf][16 * dt + cl][32 * kc + 4 * kg]);
        const uint2 hi = *reinterpret_cast<const uint2 *>(&s_vt[vbuf][16 * dt + cl][32 * kc + 16 + 4 * kg]);
        const bf16x8s vf = __builtin_bit_cast(bf16x8s, make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
        for (int ct = 0; ct < kFaCT; ++ct)
          acc[ct][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, p[ct][kc], acc[ct][dt], 0, 0, 0);
      }
  };
  // the weights of one tile as bf16 MFMA operands: a lane's 8 k-values are
  // its 4 + 4 exponentials of two S^T tiles
  bf16x8s pb[kFaCT][2], pbp[kFaCT][2];
#pragma unroll
  for (int ct = 0; ct < kFaCT; ++ct)
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) pbp[ct][kc] = __builtin_bit_cast(bf16x8s, make_uint4(0u, 0u, 0u, 0u));
  auto weights = [&](const floatx4s (&sa)[kFaCT][4]) {
#pragma unroll
    for (int ct = 0; ct < kFaCT; ++ct)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const floatx4s &a0 = sa[ct][2 * kc], &a1 = sa[ct][2 * kc + 1];
        pb[ct][kc] = bf16x8s{(__bf16)seg_exp2(a0[0]), (__bf16)seg_exp2(a0[1]), (__bf16)seg_exp2(a0[2]),
                             (__bf16)seg_exp2(a0[3]), (__bf16)seg_exp2(a1[0]), (__bf16)seg_exp2(a1[1]),
                             (__bf16)seg_exp2(a1[2]), (__bf16)seg_exp2(a1[3])};
      }
  };
  // V buffer of the tile whose PV product is pending, and whether one is.  A
  // wave's first visible tile is the sweep's first tile, and the product it
  // takes then is zero weights times the zeroed buffer 2; once a wave is
  // past its last visible entry it stays past it.
  int vprev = 2;
  bool pend = false;
  for (int t = t0; t < ntile; ++t) {
    const int buf = (t - t0) & 1, vbuf = (t - t0) % 3;
    if (t + 1 < ntile) gload(t + 1);
    if (t + 2 < ntile) pidx(t + 2);
    const int T0 = t * kFaKT;
    if (T0 <= wave_lim) {
      floatx4s sacc[kFaCT][4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        bf16x8s kf[KC];
#pragma unroll
        for (int c = 0; c < KC; ++c)
          kf[c] = __builtin_bit_cast(bf16x8s,
                                     *reinterpret_cast<const uint4 *>(&s_k[buf][16 * tt + cl][32 * c + 8 * kg]));
#pragma unroll
        for (int ct = 0; ct < kFaCT; ++ct) {
          floatx4s sa = floatx4s{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < KC; ++c) sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[c], qf[ct][c], sa, 0, 0, 0);
          sacc[ct][tt] = sa;
        }
      }
      const bool diag = T0 + kFaKT - 1 > wave_lo;            // wave-uniform
#pragma unroll
      for (int ct = 0; ct < kFaCT; ++ct) {
        if (diag) {
          // entry T0 + 16 tt + 4 kg + j is visible while <= lim
          const int rel = lim[ct] - T0 - 4 * kg;
#pragma unroll
          for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (16 * tt + j > rel) sacc[ct][tt][j] = -INFINITY;
        }
        if (W > 0) {
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            const int4 pe = *reinterpret_cast<const int4 *>(&s_pos[buf][16 * tt + 4 * kg]);
            const int pj4[4] = {pe.x, pe.y, pe.z, pe.w};
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (pj4[j] < wlo[ct]) sacc[ct][tt][j] = -INFINITY;
          }
        }
      }
      // The previous tile's PV product and this tile's exponents against the
      // current reference, their column maxima and weights, written out in
      // 2 * NT chunks whose order the compiler keeps (scheduling barriers):
      // each chunk issues the V fragment reads two PV steps ahead, one PV
      // step (one MFMA per column tile; the first 2 * kFaCT chunks also one
      // weight-sum MFMA) and EPS softmax elements, so the VALU works while the
      // matrix core multiplies.
      float mx[kFaCT];
      bool up[kFaCT];
#pragma unroll
      for (int ct = 0; ct < kFaCT; ++ct) mx[ct] = -INFINITY;
      {
        uint2 vlo[2 * NT], vhi[2 * NT];
        auto vread = [&](int k) {
          const int dt = k >> 1, kc = k & 1;
          vlo[k] = *reinterpret_cast<const uint2 *>(&s_vt[vprev][16 * dt + cl][32 * kc + 4 * kg]);
          vhi[k] = *reinterpret_cast<const uint2 *>(&s_vt[vprev][16 * dt + cl][32 * kc + 16 + 4 * kg]);
        };
        float ex[kFaCT][4][4];
        vread(0);
        vread(1);
        // softmax elements EPS k .. EPS k + EPS - 1 of the lane's 16 per
        // column tile go with PV step k
        constexpr int EPS = 16 * kFaCT / (2 * NT);
#pragma unroll
        for (int k = 0; k < 2 * NT; ++k) {
          __builtin_amdgcn_sched_barrier(0);
          if (k + 2 < 2 * NT) vread(k + 2);
          if (k < 2 * kFaCT)
            lacc[k >> 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pbp[k >> 1][k & 1], lacc[k >> 1], 0, 0, 0);
          const int dt = k >> 1, kc = k & 1;
          const bf16x8s vf = __builtin_bit_cast(bf16x8s, make_uint4(vlo[k].x, vlo[k].y, vhi[k].x, vhi[k].y));
#pragma unroll
          for (int ct = 0; ct < kFaCT; ++ct)
            acc[ct][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pbp[ct][kc], acc[ct][dt], 0, 0, 0);
#pragma unroll
          for (int u = 0; u < EPS; ++u) {
            const int e = EPS * k + u, ct = e >> 4, tt = (e & 15) >> 2, j = e & 3;
            const float v = fmaf(sacc[ct][tt][j], scale, nref[ct]);
            sacc[ct][tt][j] = v;
            mx[ct] = fmaxf(mx[ct], v);
            ex[ct][tt][j] = seg_exp2(v);
            if ((e & 7) == 7) {
              // the 8 weights of operand pb[ct][kc2]: S^T tiles 2 kc2 and 2 kc2 + 1
              const int kc2 = (e & 15) >> 3;
              const float *a0 = ex[ct][2 * kc2], *a1 = ex[ct][2 * kc2 + 1];
              pb[ct][kc2] = bf16x8s{(__bf16)a0[0], (__bf16)a0[1], (__bf16)a0[2], (__bf16)a0[3],
                                    (__bf16)a1[0], (__bf16)a1[1], (__bf16)a1[2], (__bf16)a1[3]};
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int ct = 0; ct < kFaCT; ++ct) up[ct] = mx[ct] > thr[ct];
      // (kept here, next to the MFMAs, rather than sunk past the branch below)
#pragma unroll
      for (int ct = 0; ct < kFaCT; ++ct)
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) asm volatile("" ::"v"(pb[ct][kc]));
      // A column's reference moves only if one of its four lanes sees an
      // exponent above the threshold (rare): then the column maxima are
      // reduced across the lane rows, the exponents shift, the weights are
      // taken again, and what the column has accumulated -- the previous
      // tile included -- is scaled (by 0 on its first visible tile).
      bool any_up = false;
#pragma unroll
      for (int ct = 0; ct < kFaCT; ++ct) any_up = any_up || up[ct];
      if (__any(any_up)) {
#pragma unroll
        for (int ct = 0; ct < kFaCT; ++ct) {
          mx[ct] = fa_rows_max(mx[ct]);
          up[ct] = mx[ct] > thr[ct];
          const float sh = up[ct] ? mx[ct] : 0.f;
          const float alpha = !up[ct] ? 1.f : (thr[ct] == -INFINITY ? 0.f : seg_exp2(-sh));
          nref[ct] -= sh;
          if (up[ct]) thr[ct] = AKV_FA_TAU;
#pragma unroll
          for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int j = 0; j < 4; ++j) sacc[ct][tt][j] -= sh;
          lacc[ct] *= alpha;
#pragma unroll
          for (int dt = 0; dt < NT; ++dt) acc[ct][dt] *= alpha;
        }
        weights(sacc);
      }
#pragma unroll
      for (int ct = 0; ct < kFaCT; ++ct)
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) pbp[ct][kc] = pb[ct][kc];
      vprev = vbuf;
      pend = true;
    } else if (pend) {
      // past this wave's last visible entry: the pending product, while its
      // V tile is still in LDS (the next iteration overwrites that buffer)
      pv_tile(pbp, vprev);
      pend = false;
    }
    if (t + 1 < ntile) lstore(t + 1, buf ^ 1, (t + 1 - t0) % 3);
    __syncthreads();
  }
  if (pend) pv_tile(pbp, vprev);

#pragma unroll
  for (int ct = 0; ct < kFaCT; ++ct) {
    if (!rok[ct]) continue;
    const float inv = cok[ct] ? 1.f / lacc[ct][0] : 0.f;   // an invalid segment's rows are zero
    uint16_t *orow = out + qrow[ct] * D + 4 * kg;
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) {
      const uint32_t w0 = (uint16_t)seg_bf16(acc[ct][dt][0] * inv) |
                          ((uint32_t)(uint16_t)seg_bf16(acc[ct][dt][1] * inv) << 16);
      const uint32_t w1 = (uint16_t)seg_bf16(acc[ct][dt][2] * inv) |
                          ((uint32_t)(uint16_t)seg_bf16(acc[ct][dt][3] * inv) << 16);
      *reinterpret_cast<uint2 *>(orow + 16 * dt) = make_uint2(w0, w1);
    }
  }
}

hipError_t launch_segment_attention(const Dev &d, const uint16_t *q, const int32_t *seg_seq,
                                    const int32_t *seg_q_off, int n_seg, int max_q, int l0,
                                    int nL, int Hq, uint16_t *out, hipStream_t st) {
  const int G = Hq / d.H;
  const int TB = 16 / G;
  const dim3 block(kSegWaves * 64);
  if (max_q > TB) {
    // more rows than one 16-column tile holds: the prefill-shaped kernel
    const int TBW = kFaCols / G;
    const dim3 grid((max_q + TBW - 1) / TBW, n_seg, nL * d.H), fblock(kFaWaves * 64);
    if (d.D == 128)
      hipLaunchKernelGGL(segment_fa_kernel<128>, grid, fblock, 0, st, d, q, seg_seq, seg_q_off,
                         max_q, l0, nL, Hq, out);
    else
      hipLaunchKernelGGL(segment_fa_kernel<64>, grid, fblock, 0, st, d, q, seg_seq, seg_q_off,
                         max_q, l0, nL, Hq, out);
    return hipGetLastError();
  }
  const dim3 grid((max_q + TB - 1) / TB, n_seg, nL * d.H);
  if (d.D == 128)
    hipLaunchKernelGGL(segment_attn_kernel<128>, grid, block, 0, st, d, q, seg_seq, seg_q_off,
                       max_q, l0, nL, Hq, out);
  else
    hipLaunchKernelGGL(segment_attn_kernel<64>, grid, block, 0, st, d, q, seg_seq, seg_q_off,
                       max_q, l0, nL, Hq, out);
  return hipGetLastError();
}

}  // namespace akv
