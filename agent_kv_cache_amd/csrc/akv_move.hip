// Move / re-rotate kernel of libakv for gfx950 ([CE] sec. 3.3 eqs. 4-5;
// [AKV] sec. 5.5: the reposition kernel un-rotates at p and rotates to q,
// copies when p == q, copies V and never rotates it, and writes to a
// separate destination slot).
//
// A persistent grid walks (page, layer) units of the rebuilt pages.  Pages
// from the first dropped page on are rebuilt out of place in fresh pages (K
// re-rotated when its delta is non-zero, V copied bitwise); pages before it
// whose positions change are re-rotated in place.  16-B loads and stores, one
// (row, 8 NeoX pairs) per thread.  The same kernel serves akv_fork (every
// page of the copy rebuilt, sources left untouched).
#include "akv_internal.h"
#include "akv_rope.h"

namespace akv {

// Launch-shape knobs of the move kernel (compile-time; defaults are the
// measured best on MI355X for the configurations of the benchmark).
#ifndef AKV_MOVE_UNROLL
#define AKV_MOVE_UNROLL 2      // (layer, head) slices loaded before any store
#endif
#ifndef AKV_MOVE_MIN_WAVES
#define AKV_MOVE_MIN_WAVES 4   // waves per SIMD the register budget must allow
#endif
#ifndef AKV_MOVE_NT
#define AKV_MOVE_NT 1          // nontemporal hint on the streamed KV accesses
#endif
#ifndef AKV_MOVE_SPLIT_KV
#define AKV_MOVE_SPLIT_KV 1    // stream a unit's K slices, then its V slices
#endif
#ifndef AKV_MOVE_ROTATE
#define AKV_MOVE_ROTATE 0      // start each page's layer walk at a page-dependent layer
#endif

constexpr int kMoveThreads = 256;

// Streaming 16-B accesses: every KV byte of a move is read once and written
// once, so they bypass cache retention (nontemporal hint) -- when each load
// instruction covers whole 128-B lines.  With partial RoPE a row's x and y
// chunks are two 64-B pieces per instruction; the other half of each line is
// touched by the next instruction, and with the hint it is fetched again, so
// those moves use ordinary cached accesses (measured 1.05 -> 0.89 ms on the
// Llama-8B-shaped drop with r = 64).
template <bool NT>
__device__ __forceinline__ u32x4 ld_stream(const uint16_t *p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  else return *reinterpret_cast<const u32x4 *>(p);
}
template <bool NT>
__device__ __forceinline__ void st_stream(uint16_t *p, u32x4 v) {
  if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
  else *reinterpret_cast<u32x4 *>(p) = v;
}

// Work split: the rebuilt pages (moved first, then in-place) times the L
// layers form U = pages * L (page, layer) units, ordered page-major.  Workgroup
// w takes the contiguous units [w*U/G, (w+1)*U/G), so every workgroup moves
// the same number of (layer, page) slices whatever the page count, and the
// per-page set-up (row sources, deltas, cos/sin) is done once per page it
// touches.
template <int D, bool NT>
__global__ __launch_bounds__(kMoveThreads, AKV_MOVE_MIN_WAVES) void move_kernel(Dev d, int mode) {
  constexpr int HALF = D / 2;
  constexpr int CH = D / 16;             // 16-B chunks per half row
  constexpr int TPH = kPage * CH;        // threads per (layer, head) slice
  constexpr int NS = kMoveThreads / TPH; // slices per pass
  constexpr int U = AKV_MOVE_UNROLL;      // slices loaded before any store
  __shared__ int s_b, s_po, s_dst, s_mv;
  __shared__ int s_src[kPage], s_valid[kPage], s_delta[kPage], s_rep[kPage];
  __shared__ int s_repval[kPage], s_nrep;
  __shared__ double2 s_cs[kPage][HALF];

  if (d.ctl[CTL_OP_OK] == 0) return;
  const int Tm = d.ctl[CTL_T_MOVE], Ti = d.ctl[CTL_T_INPLACE];
  const long long npages = (long long)Tm + Ti;
  if (npages == 0) return;
  const int fc_old = d.ctl[CTL_FC_OLD];
  const long long units = npages * d.L;
  const long long u0 = units * blockIdx.x / gridDim.x;
  const long long u1 = units * (blockIdx.x + 1) / gridDim.x;
  const int t = threadIdx.x;
  const int r = (t % TPH) / CH, pc = t % CH, slot = t / TPH;
  // Chunk pc of a row: a rotary chunk pairs dims [8pc, 8pc+8) with the same
  // dims + RD/2; past the rotary part ([RD, D), partial RoPE) chunks are only
  // copied, paired the same way over the tail.
  const int rch = d.RD / 16;
  const bool rot_chunk = pc < rch;
  const int xo = rot_chunk ? 8 * pc : d.RD + 8 * (pc - rch);
  const int yoff = rot_chunk ? d.RD / 2 : (D - d.RD) / 2;
  const size_t S = (size_t)d.S;
  const PoolStrides ps = pool_strides(d.NB, d.H, D);
  const size_t hstride = ps.head, lstride = ps.layer;
  const bool rot_any = (mode & M_REPOS) != 0;

  for (long long pgl = u0 / d.L; pgl * d.L < u1; ++pgl) {
    const int pg = (int)pgl;
    const int l0 = (int)(max(u0, pgl * d.L) - pgl * d.L);
    const int l1 = (int)(min(u1, (pgl + 1) * d.L) - pgl * d.L);
    __syncthreads();  // LDS of the previous page is no longer read
    if (t == 0) {
      const bool mv = pg < Tm;
      const int key = mv ? pg : pg - Tm;
      const int of = mv ? SI_MOVE_OFF : SI_INPLACE_OFF;
      int lo = 0, hi = d.B - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (d.seq_info[(size_t)mid * kSeqInfo + of] <= key) lo = mid; else hi = mid - 1;
      }
      const int *si = d.seq_info + (size_t)lo * kSeqInfo;
      const int po = (mv ? si[SI_FBD] : si[SI_FIP]) + (key - si[of]);
      s_b = lo;
      s_po = po;
      s_mv = mv;
      s_dst = mv ? d.free_stack[fc_old - 1 - pg] : d.table[(size_t)lo * d.maxpg + po];
      if (mv && l0 == 0) d.stage[pg] = s_dst;
    }
    __syncthreads();
    const int b = s_b, po = s_po, dst = s_dst;
    const bool mv = s_mv;
    if (t < kPage) {
      const int rnew = d.seq_info[(size_t)b * kSeqInfo + SI_NEW_LEN];
      const int j = po * kPage + t;
      const bool valid = j < rnew;
      // physical source slot (page * 16 + row); in place: the slot itself
      const int src = !valid ? 0
                      : ((mv && (mode & (M_DROP | M_FORK))) ? d.src_map[b * S + j]
                                                 : d.table[(size_t)b * d.maxpg + po] * kPage + t);
      const int delta = (valid && (mode & M_REPOS)) ? d.delta_map[b * S + j] : 0;
      s_src[t] = src;
      s_valid[t] = valid;
      s_delta[t] = delta;
      if (l0 == 0) {
        const size_t dn = (size_t)dst * kPage + t;
        if (mv) {
          d.pos[dn] = valid ? d.pos[src] + delta : -1;
          d.tok[dn] = valid ? d.tok[src] : -1;
        } else if (valid && delta != 0) {
          d.pos[dn] += delta;
        }
      }
    }
    __syncthreads();
    if (rot_any) {
      if (t == 0) {
        int n = 0;
        for (int rr = 0; rr < kPage; ++rr) {
          const int dl = s_delta[rr];
          int k = 0;
          while (k < n && s_repval[k] != dl) ++k;
          if (k == n) s_repval[n++] = dl;
          s_rep[rr] = k;
        }
        s_nrep = n;
      }
      __syncthreads();
      const int RH = d.RD / 2;
      const int ntask = s_nrep * RH;
      for (int task = t; task < ntask; task += kMoveThreads) {
        const int ri = task / RH, i = task - ri * RH;
        const int dl = s_repval[ri];
        double sn = 0.0, cs = 1.0;
        if (dl != 0) sincos((double)dl * d.theta[i], &sn, &cs);
        s_cs[ri][i] = make_double2(cs, sn);
      }
      __syncthreads();
    }
    const bool valid = s_valid[r] != 0;
    const int delta = s_delta[r];
    // cos/sin of this thread's 8 pairs stay in LDS and are read per use
    const double2 *cs_row = &s_cs[(rot_any && delta != 0) ? s_rep[r] : 0][rot_chunk ? 8 * pc : 0];
    const bool turn = valid && delta != 0 && rot_chunk;
    const bool do_k = valid ? (mv || turn) : mv;
    const bool do_v = mv;
    if (!do_k) continue;
    const int nsl = (l1 - l0) * d.H;
#if AKV_MOVE_ROTATE
    // the k-th unit of page pg is layer (k + rot) mod L: concurrently
    // running workgroups then stream different layers' regions
    const int rot = (int)((pgl * 7) % d.L);
#endif
    const int sp = s_src[r];
    const size_t src_row = (size_t)(sp >> 4) * ps.page + (size_t)(sp & 15) * D + xo;
    const size_t dst_row = (size_t)dst * ps.page + (size_t)r * D + xo;
#if AKV_MOVE_SPLIT_KV
    // K slices of the unit range first, then V slices: each pass streams one
    // pool (two concurrent streams per workgroup instead of four)
    for (int plane = 0; plane < (do_v ? 2 : 1); ++plane) {
      uint16_t *pool = plane ? d.v : d.k;
      const bool rot_plane = plane == 0 && turn;
      for (int i0 = slot; i0 < nsl; i0 += NS * U) {
        u32x4 lo[U], hi[U];
        size_t dofs[U];
        bool on[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int idx = i0 + u * NS;
          on[u] = idx < nsl;
          const int l = l0 + idx / d.H, h = idx % d.H;
          const size_t off = (size_t)l * lstride + (size_t)h * hstride;
          dofs[u] = dst_row + off;
          lo[u] = hi[u] = u32x4{0u, 0u, 0u, 0u};
          if (on[u] && valid) {
            lo[u] = ld_stream<NT>(pool + src_row + off);
            hi[u] = ld_stream<NT>(pool + src_row + off + yoff);
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (!on[u]) continue;
          if (rot_plane) rotate8(lo[u], hi[u], cs_row);
          st_stream<NT>(pool + dofs[u], lo[u]);
          st_stream<NT>(pool + dofs[u] + yoff, hi[u]);
        }
      }
    }
#else
    for (int i0 = slot; i0 < nsl; i0 += NS * U) {
      u32x4 klo[U], khi[U], vlo[U], vhi[U];
      size_t dofs[U];
      bool on[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int idx = i0 + u * NS;
        on[u] = idx < nsl;
#if AKV_MOVE_ROTATE
        int l = l0 + idx / d.H + rot;
        if (l >= d.L) l -= d.L;
#else
        const int l = l0 + idx / d.H;
#endif
        const int h = idx % d.H;
        const size_t off = (size_t)l * lstride + (size_t)h * hstride;
        dofs[u] = dst_row + off;
        klo[u] = khi[u] = vlo[u] = vhi[u] = u32x4{0u, 0u, 0u, 0u};
        if (on[u] && valid) {
          const size_t so = src_row + off;
          klo[u] = ld_stream<NT>(d.k + so);
          khi[u] = ld_stream<NT>(d.k + so + yoff);
          if (do_v) {
            vlo[u] = ld_stream<NT>(d.v + so);
            vhi[u] = ld_stream<NT>(d.v + so + yoff);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (!on[u]) continue;
        if (turn) rotate8(klo[u], khi[u], cs_row);
        st_stream<NT>(d.k + dofs[u], klo[u]);
        st_stream<NT>(d.k + dofs[u] + yoff, khi[u]);
        if (do_v) {
          st_stream<NT>(d.v + dofs[u], vlo[u]);
          st_stream<NT>(d.v + dofs[u] + yoff, vhi[u]);
        }
      }
    }
#endif
  }
}

hipError_t launch_move(const Dev &d, int mode, int grid, hipStream_t st) {
  const bool nt = AKV_MOVE_NT && d.RD == d.D;
  const dim3 g(grid), b(kMoveThreads);
  if (d.D == 128) {
    if (nt) hipLaunchKernelGGL((move_kernel<128, true>), g, b, 0, st, d, mode);
    else hipLaunchKernelGGL((move_kernel<128, false>), g, b, 0, st, d, mode);
  } else {
    if (nt) hipLaunchKernelGGL((move_kernel<64, true>), g, b, 0, st, d, mode);
    else hipLaunchKernelGGL((move_kernel<64, false>), g, b, 0, st, d, mode);
  }
  return hipGetLastError();
}

int move_blocks_per_cu(int D) {
  int n = 0;
  const hipError_t e = (D == 128)
      ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, move_kernel<128, true>, kMoveThreads, 0)
      : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, move_kernel<64, true>, kMoveThreads, 0);
  return (e == hipSuccess && n > 0) ? n : 2;
}

}  // namespace akv
