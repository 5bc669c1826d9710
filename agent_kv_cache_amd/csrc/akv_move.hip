// Move / re-rotate kernel of libakv for gfx950 ([CE] sec. 3.3 eqs. 4-5;
// [AKV] sec. 5.5: the reposition kernel un-rotates at p and rotates to q,
// copies when p == q, copies V and never rotates it, and writes to a
// separate destination slot).
//
// The kernel walks (page, layer) units of the rebuilt pages.  Pages from the
// first dropped page on are rebuilt out of place in fresh pages (K re-rotated
// when its delta is non-zero, V copied bitwise); pages before it whose
// positions change are re-rotated in place.  16-B loads and stores, one
// (row, 8 NeoX pairs) per thread.  The same kernel serves akv_fork (every
// page of the copy rebuilt, sources left untouched).
//
// Two launch shapes, chosen on the device from the planned unit count:
//  * one-shot (ops of up to 131072 blocks): one block per page and layer
//    group (one layer) in layer-major order.
//    Blocks are dispatched in index order, so the blocks in flight read and
//    write a compact, sliding address range; on MI355X this streams ~15%
//    faster than a persistent grid whose workgroups each walk their own
//    pages through all layers (measured on the Llama-8B-shaped drop: 0.87 ->
//    0.74 ms).
//  * persistent (larger ops): occupancy x CUs workgroups, each taking a
//    contiguous range of page-major units, so the per-page set-up is shared
//    by all the layers a workgroup moves.
#include "akv_internal.h"
#include "akv_rope.h"

namespace akv {

// Launch-shape knobs of the move kernel (compile-time; defaults are the
// measured best on MI355X for the configurations of the benchmark).
#ifndef AKV_MOVE_UNROLL
#define AKV_MOVE_UNROLL 2      // (layer, head) slices loaded before any store (one-shot grid)
#endif
#ifndef AKV_MOVE_UNROLL_PERSIST
#define AKV_MOVE_UNROLL_PERSIST 1  // the same for the persistent grid
#endif
#ifndef AKV_MOVE_MIN_WAVES
#define AKV_MOVE_MIN_WAVES 4   // waves per SIMD the register budget must allow
#endif
#ifndef AKV_MOVE_NT
#define AKV_MOVE_NT 1          // nontemporal hint on the streamed KV accesses
#endif
#ifndef AKV_MOVE_FR64
#define AKV_MOVE_FR64 1        // full-row thread mapping at d = 64
#endif
#ifndef AKV_MOVE_FR_PARTIAL
#define AKV_MOVE_FR_PARTIAL 1  // full-row thread mapping for partial RoPE
#endif
#ifndef AKV_MOVE_FR_NT
#define AKV_MOVE_FR_NT 1       // nontemporal hint with the full-row mapping
#endif
#ifndef AKV_MOVE_FR_ITEMS
#define AKV_MOVE_FR_ITEMS 4    // full-row mapping: (plane, slice) items loaded before any store
#endif

constexpr int kMoveThreads = 256;

// Streaming 16-B accesses: every KV byte of a move is read once and written
// once, so they bypass cache retention (nontemporal hint) -- when each load
// instruction covers whole 128-B lines, i.e. full RoPE at d = 128.  Otherwise
// (partial RoPE, or d = 64 where a half row is 64 B) a row's x and y chunks
// are two 64-B pieces per instruction; the other half of each line is touched
// by the next instruction, and with the hint it is fetched again, so those
// moves use ordinary cached accesses (measured: Llama-8B-shaped drop with
// r = 64 1.05 -> 0.89 ms; the d = 64 history ops 4.0 -> 4.17 TB/s).
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
// layers form U = pages * L (page, layer) units.  Persistent launch: units
// ordered page-major, workgroup w takes the contiguous units
// [w*U/G, (w+1)*U/G), so every workgroup moves the same number of (layer,
// page) slices whatever the page count, and the per-page set-up (row
// sources, deltas, cos/sin) is done once per page it touches.  One-shot
// launch: block b takes page b mod pages at layer group b / pages.
//
// Thread mapping.  Half rows (FR = false; full RoPE at d = 128): a thread
// holds chunk pc of the x half of a row and the matching chunk of the y half
// (8 NeoX pairs), loaded by two instructions that each cover whole 128-B
// lines.  Full rows (FR = true; d = 64, where a row is one line, and partial
// RoPE, where x and y chunks are 64-B pieces): a thread holds one chunk c of
// the row, so every load instruction covers whole lines; a rotary chunk's
// partner (c +- r/16) is read from the lane that holds it (the same row's
// lanes are adjacent), tail chunks are only copied.
template <int D, bool NT, bool ONESHOT, bool FR>
__device__ __forceinline__ void move_body(const Dev &d, int mode, int oneshot_cap, int group) {
  constexpr int HALF = D / 2;
  constexpr int CH = D / 16;             // 16-B chunks per half row
  constexpr int CPR = FR ? 2 * CH : CH;  // threads per row
  constexpr int TPH = kPage * CPR;       // threads per (layer, head) slice
  constexpr int NS = kMoveThreads / TPH; // slices per pass
  // (plane, slice) items loaded before any store (a full-row thread holds
  // half the bytes of a half-row thread per item, so it takes more)
  constexpr int U = FR ? AKV_MOVE_FR_ITEMS : ONESHOT ? AKV_MOVE_UNROLL : AKV_MOVE_UNROLL_PERSIST;
  __shared__ int s_dst, s_mv;
  __shared__ int s_src[kPage], s_valid[kPage], s_delta[kPage], s_rep[kPage];
  __shared__ int s_repval[kPage], s_nrep;
  __shared__ double2 s_cs[kPage][HALF];

  constexpr int LPB = AKV_MOVE_OS_LAYERS > 0 ? AKV_MOVE_OS_LAYERS : (D == 128 ? 1 : 2);
  const long long ngroups = (d.L + LPB - 1) / LPB;
  if (group == 0) {
    // One load decides for the blocks with nothing to do (an op's one-shot
    // grid is sized for the largest op the cache can plan, so most of its
    // blocks usually leave here): the pages of group 0, 0 when nothing moves.
    const long long np0 = d.ctl[CTL_NPG0];
    if (np0 == 0 || (np0 * ngroups <= oneshot_cap) != ONESHOT) return;
    if (ONESHOT && blockIdx.x >= np0 * ngroups) return;
  } else if (group >= d.ctl[CTL_NGROUPS]) {
    return;
  }
  // this round's group of sequences: its moved pages take the fresh pages
  // below the group's free count, its rebuilt pages are numbered from 0
  const int *gr = d.groups + (size_t)group * kGroupRec;
  const int Tm = gr[GR_TM], Ti = gr[GR_TI];
  const long long npages = (long long)Tm + Ti;
  if (npages == 0) return;
  const int fc_old = gr[GR_FC], moff = gr[GR_MOFF], ioff = gr[GR_IOFF];
  const long long units = npages * d.L;
  // Two launches share the work.  An op of at most oneshot_cap blocks runs in
  // the one-shot launch: one block per LPB layers of a page, in layer-major
  // order -- block b moves page b mod pages at layer group b / pages -- so
  // the blocks in flight cover a compact address range.  A larger op runs in
  // the persistent launch (contiguous unit ranges).  One-shot blocks move
  // LPB consecutive layers (64 KiB of K+V read per block at the Llama-8B
  // shape, whatever the head size; blocks per (page, layer, plane) or per
  // head group were measured slower: each repeats the per-page set-up).
  const long long os_blocks = npages * ngroups;
  if ((os_blocks <= oneshot_cap) != ONESHOT) return;
  long long u0, u1;
  if (ONESHOT) {
    if (blockIdx.x >= os_blocks) return;
    const long long pg = blockIdx.x % npages, lg = blockIdx.x / npages;
    u0 = pg * d.L + lg * LPB;
    u1 = min(u0 + LPB, (pg + 1) * d.L);
  } else {
    u0 = units * blockIdx.x / gridDim.x;
    u1 = units * (blockIdx.x + 1) / gridDim.x;
  }
  const int t = threadIdx.x;
  const int r = (t % TPH) / CPR, pc = t % CPR, slot = t / TPH;
  // Half rows: chunk pc of a row, a rotary chunk pairs dims [8pc, 8pc+8)
  // with the same dims + RD/2; past the rotary part ([RD, D), partial RoPE)
  // chunks are only copied, paired the same way over the tail.  Full rows:
  // chunk pc holds dims [8pc, 8pc+8); chunks below RD/8 are rotary, an x
  // chunk when pc < RD/16 (partner pc + RD/16), else a y chunk (partner
  // pc - RD/16).
  const int rch = d.RD / 16;
  const bool rot_chunk = FR ? pc < 2 * rch : pc < rch;
  const bool x_chunk = pc < rch;
  const int xo = (FR || rot_chunk) ? 8 * pc : d.RD + 8 * (pc - rch);
  const int yoff = FR ? 0 : rot_chunk ? d.RD / 2 : (D - d.RD) / 2;
  const int partner_lane = (int)(threadIdx.x & 63) + (x_chunk ? rch : -rch);
  const size_t S = (size_t)d.S;
  const PoolStrides ps = pool_strides(d.NB, d.H, D);
  const size_t hstride = ps.head, lstride = ps.layer;
  const bool rot_any = (mode & M_REPOS) != 0;

  for (long long pgl = u0 / d.L; pgl * d.L < u1; ++pgl) {
    const int pg = (int)pgl;
    const int l0 = (int)(max(u0, pgl * d.L) - pgl * d.L);
    const int l1 = (int)(min(u1, (pgl + 1) * d.L) - pgl * d.L);
    __syncthreads();  // LDS of the previous page is no longer read
    // Rows: the 16 lanes t < 16 of wave 0 each find the page's sequence and
    // destination (the same loads in every lane) and their row's source slot
    // and delta, then rank the page's distinct deltas among themselves.
    if (t < kPage) {
      const bool mv = pg < Tm;
      const int key = mv ? moff + pg : ioff + (pg - Tm);   // global offsets over sequences
      const int of = mv ? SI_MOVE_OFF : SI_INPLACE_OFF;
      int lo = 0, hi = d.B - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (d.seq_info[(size_t)mid * kSeqInfo + of] <= key) lo = mid; else hi = mid - 1;
      }
      const int b = lo;
      const int *si = d.seq_info + (size_t)b * kSeqInfo;
      const int po = (mv ? si[SI_FBD] : si[SI_FIP]) + (key - si[of]);
      // fresh page: popped from the free stack (or, staged by the plan, read
      // from the staging array); in place: the page itself
      const int dst = !mv ? d.table[(size_t)b * d.maxpg + po]
                      : (mode & M_STAGED) ? d.stage[moff + pg] : d.free_stack[fc_old - 1 - pg];
      const int j = po * kPage + t;
      const bool valid = j < si[SI_NEW_LEN];
      // physical source slot (page * 16 + row); in place: the slot itself
      const int src = !valid ? 0
                      : ((mv && (mode & (M_DROP | M_FORK))) ? d.src_map[b * S + j]
                                                             : d.table[(size_t)b * d.maxpg + po] * kPage + t);
      const int delta = (valid && (mode & M_REPOS)) ? d.delta_map[b * S + j] : 0;
      s_src[t] = src;
      s_valid[t] = valid;
      s_delta[t] = delta;
      if (t == 0) {
        s_dst = dst;
        s_mv = mv;
        if (mv && l0 == 0 && !(mode & M_STAGED)) d.stage[moff + pg] = dst;
      }
      if (l0 == 0) {
        const size_t dn = (size_t)dst * kPage + t;
        if (mv) {
          d.pos[dn] = valid ? d.pos[src] + delta : -1;
          d.tok[dn] = valid ? d.tok[src] : -1;
        } else if (valid && delta != 0) {
          d.pos[dn] += delta;
        }
      }
      if (rot_any) {
        // slot of a delta = the number of distinct deltas whose first row
        // comes earlier (lanes 0..15 of wave 0 are the rows)
        int first = t;
        for (int rr = kPage - 1; rr >= 0; --rr)
          if (__shfl(delta, rr, 64) == delta) first = rr;
        const bool is_first = first == t;
        const unsigned long long fm = __ballot(is_first) & 0xFFFFull;
        const int rep = __popcll(fm & ((1ull << first) - 1ull));
        s_rep[t] = rep;
        if (is_first) s_repval[rep] = delta;
        if (t == 0) s_nrep = __popcll(fm);
      }
    }
    __syncthreads();
    const bool mv = s_mv;
    const int dst = s_dst;
    const bool valid = s_valid[r] != 0;
    const int delta = s_delta[r];
    const bool turn = valid && delta != 0 && rot_chunk;
    const bool do_k = valid ? (mv || turn) : mv;
    const int pend = mv ? 2 : 1;   // planes: K, and V when the page moves
    const int nsl = (l1 - l0) * d.H;
    const int sp = s_src[r];
    const size_t src_row = (size_t)(sp >> 4) * ps.page + (size_t)(sp & 15) * D + xo;
    const size_t dst_row = (size_t)dst * ps.page + (size_t)r * D + xo;
    // Items: the (plane, slice) pairs of the unit range, K slices first,
    // then V slices, taken in batches of U per thread (a batch may hold both
    // planes).  The first batch is loaded before the cos/sin set-up so that
    // its latency covers the set-up.
    const int nit = do_k ? pend * nsl : 0;
    int i0 = slot;
    u32x4 lo[U], hi[U];
    size_t dofs[U];
    bool on[U], kp[U];
    auto issue = [&]() {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int idx = i0 + u * NS;
        on[u] = idx < nit;
        kp[u] = idx < nsl;
        const int sl = kp[u] ? idx : idx - nsl;
        const int l = l0 + sl / d.H, h = sl % d.H;
        const size_t off = (size_t)l * lstride + (size_t)h * hstride;
        dofs[u] = dst_row + off;
        lo[u] = hi[u] = u32x4{0u, 0u, 0u, 0u};
        if (on[u] && valid) {
          const uint16_t *pool = kp[u] ? d.k : d.v;
          lo[u] = ld_stream<NT>(pool + src_row + off);
          if constexpr (!FR) hi[u] = ld_stream<NT>(pool + src_row + off + yoff);
        }
      }
    };
    if (i0 < nit) issue();
    if (rot_any) {
      const int RH = d.RD / 2;
      const int ntask = s_nrep * RH;
      for (int task = t; task < ntask; task += kMoveThreads) {
        const int ri = task / RH, i = task - ri * RH;
        const int dl = s_repval[ri];
        double sn = 0.0, cs = 1.0;
        if (dl != 0) sincos_rope((double)dl * d.theta[i], &sn, &cs);
        s_cs[ri][i] = make_double2(cs, sn);
      }
      __syncthreads();
    }
    // cos/sin of this thread's 8 pairs stay in LDS and are read per use
    const double2 *cs_row = &s_cs[(rot_any && delta != 0) ? s_rep[r] : 0]
                                 [!rot_chunk ? 0 : x_chunk ? 8 * pc : 8 * (pc - rch)];
    while (i0 < nit) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (!on[u]) continue;
        uint16_t *pool = kp[u] ? d.k : d.v;
        const bool rot_plane = kp[u] && turn;
        if constexpr (FR) {
          if (rot_plane) {
            // both lanes of a pair hold the same row, so they turn together
            const u32x4 other = {(uint32_t)__shfl((int)lo[u].x, partner_lane, 64),
                                 (uint32_t)__shfl((int)lo[u].y, partner_lane, 64),
                                 (uint32_t)__shfl((int)lo[u].z, partner_lane, 64),
                                 (uint32_t)__shfl((int)lo[u].w, partner_lane, 64)};
            lo[u] = rotate8_side(lo[u], other, x_chunk, cs_row);
          }
          st_stream<NT>(pool + dofs[u], lo[u]);
        } else {
          if (rot_plane) rotate8(lo[u], hi[u], cs_row);
          st_stream<NT>(pool + dofs[u], lo[u]);
          st_stream<NT>(pool + dofs[u] + yoff, hi[u]);
        }
      }
      i0 += NS * U;
      if (i0 < nit) issue();
    }
  }
}

// The first round of an op (every op that fits the free pool at once).
template <int D, bool NT, bool ONESHOT, bool FR>
__global__ __launch_bounds__(kMoveThreads, AKV_MOVE_MIN_WAVES) void move_kernel(Dev d, int mode,
                                                                                 int oneshot_cap) {
  move_body<D, NT, ONESHOT, FR>(d, mode, oneshot_cap, 0);
}

// Later rounds of an op split into sequence groups (persistent shape).  A
// kernel of its own, so that profiles keep the first round's launches apart
// from these, which exit at once whenever the op needed fewer groups.
template <int D, bool NT, bool FR>
__global__ __launch_bounds__(kMoveThreads, AKV_MOVE_MIN_WAVES) void move_round_kernel(Dev d,
                                                                                       int mode,
                                                                                       int group) {
  move_body<D, NT, false, FR>(d, mode, 0, group);
}

// Group 0: the one-shot launch, then (grid > 0) the persistent one; each
// checks the group's unit count and only one of them moves.  Later groups (an
// op split because the free pool was short): the persistent launch alone,
// with a one-shot cap of 0 so that it always moves.
template <int D, bool NT, bool FR>
static void launch_move_pair(const Dev &d, int mode, int grid, int oneshot_cap, int group,
                             hipStream_t st) {
  const dim3 b(kMoveThreads);
  if (group == 0) {
    hipLaunchKernelGGL((move_kernel<D, NT, true, FR>), dim3(oneshot_cap), b, 0, st, d, mode,
                       oneshot_cap);
    if (grid > 0)
      hipLaunchKernelGGL((move_kernel<D, NT, false, FR>), dim3(grid), b, 0, st, d, mode,
                         oneshot_cap);
  } else {
    hipLaunchKernelGGL((move_round_kernel<D, NT, FR>), dim3(grid), b, 0, st, d, mode, group);
  }
}

// Whether a cache's moves use the full-row mapping.
static bool move_full_rows(int D, int RD) {
  return D == 64 ? AKV_MOVE_FR64 != 0 : (RD < D && AKV_MOVE_FR_PARTIAL != 0);
}

// The one-shot launch (oneshot_cap blocks), then the persistent grid (grid
// workgroups; 0 when no op of this cache can exceed the one-shot launch);
// each checks the planned unit count and only one of them moves.  Every
// mapping whose load instructions cover whole lines uses the nontemporal
// hint (half rows of full RoPE at d = 128, full rows); the half-row mapping
// of partial RoPE (64-B pieces) uses cached accesses.
hipError_t launch_move(const Dev &d, int mode, int grid, int oneshot_cap, int group,
                       hipStream_t st) {
  constexpr bool kFrNT = AKV_MOVE_FR_NT != 0;
  if (move_full_rows(d.D, d.RD)) {
    if (d.D == 128) launch_move_pair<128, kFrNT, true>(d, mode, grid, oneshot_cap, group, st);
    else launch_move_pair<64, kFrNT, true>(d, mode, grid, oneshot_cap, group, st);
  } else if (d.D == 128) {
    if (AKV_MOVE_NT && d.RD == d.D)
      launch_move_pair<128, true, false>(d, mode, grid, oneshot_cap, group, st);
    else launch_move_pair<128, false, false>(d, mode, grid, oneshot_cap, group, st);
  } else {
    launch_move_pair<64, false, false>(d, mode, grid, oneshot_cap, group, st);
  }
  return hipGetLastError();
}

int move_blocks_per_cu(int D, int RD) {
  constexpr bool kFrNT = AKV_MOVE_FR_NT != 0;
  const bool fr = move_full_rows(D, RD);
  int n = 0;
  hipError_t e;
  if (D == 128)
    e = fr ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, move_kernel<128, kFrNT, false, true>,
                                                          kMoveThreads, 0)
           : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, move_kernel<128, true, false, false>,
                                                          kMoveThreads, 0);
  else
    e = fr ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, move_kernel<64, kFrNT, false, true>,
                                                          kMoveThreads, 0)
           : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, move_kernel<64, false, false, false>,
                                                          kMoveThreads, 0);
  return (e == hipSuccess && n > 0) ? n : 2;
}

}  // namespace akv
