// Drop / reposition plan and commit, append, release and reset kernels of
// libakv for gfx950.
//
// [CE] = review of "Cache Engineering for Agents", sec. 3.3 eqs. (3)-(5);
// [AKV] = "[Repo Review] AKV", sec. 1 (drop then reposition), sec. 5.5.
//
// One drop / reposition / fork runs as three stream-ordered kernels:
//   plan   : workgroups of 256 pages per (chunk, sequence) scan the keep
//            flags (16 mask bytes per thread, one 16-B load), build the
//            gather map src[j] and the per-survivor rotation delta q - p,
//            and find the first dropped slot and the first changed position;
//            the last workgroup to finish (ticket counter) takes prefix sums
//            over sequences, checks the free pool and latches errors.
//   move   : akv_move.hip.
//   commit : new page-table entries, freed pages back on the free stack,
//            lengths and next positions.
#include "akv_internal.h"
#include "akv_rope.h"

#include <algorithm>
#include <climits>

namespace akv {

constexpr int kPlanThreads = 1024;

// Plan tickets ordered by one release fence per workgroup and one acquire in
// the last one (0: full fences around each ticket step).
#ifndef AKV_PLAN_SCOPED_FENCES
#define AKV_PLAN_SCOPED_FENCES 1
#endif

// ---------------------------------------------------------------------------
// helpers
// ---------------------------------------------------------------------------
// Exclusive block-wide prefix sum of one int per thread.  `wave_tmp` holds
// NT/64 + 1 ints of LDS.  Returns the exclusive prefix; *total gets the sum.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int x, int *wave_tmp, int *total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int v = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  if (lane == 63) wave_tmp[wid] = v;
  __syncthreads();
  if (wid == 0) {
    int w = (lane < NT / 64) ? wave_tmp[lane] : 0;
    int s = w;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int y = __shfl_up(s, o, 64);
      if (lane >= o) s += y;
    }
    if (lane < NT / 64) wave_tmp[lane] = s - w;
    if (lane == NT / 64 - 1) wave_tmp[NT / 64] = s;
  }
  __syncthreads();
  const int res = v - x + wave_tmp[wid];
  *total = wave_tmp[NT / 64];
  __syncthreads();
  return res;
}

// ---------------------------------------------------------------------------
// plan
// ---------------------------------------------------------------------------
// A sequence's pages are cut into chunks of kChunkPages pages, one 256-thread
// workgroup per (chunk, sequence) and one page per thread, so a long sequence
// is planned by many CUs, in one launch.  Each workgroup recounts the keep
// bits of its sequence's earlier chunks (the survivor rank of its first page),
// takes an in-chunk prefix sum, and writes the gather map src[j] (physical
// slot) and the rotation delta q_j - p, staged in LDS and written coalesced,
// plus its chunk's keep count and first dropped slot; the last workgroup
// finalizes every sequence and the op.
constexpr int kChunkPages = kPlanChunkPages;

__device__ __forceinline__ unsigned page_drop_bits(const uint4 m) {
  const uint32_t w[4] = {m.x, m.y, m.z, m.w};
  unsigned bits = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e) bits |= (((w[q] >> (8 * e)) & 0xFFu) != 0u) << (4 * q + e);
  return bits;
}

__device__ __forceinline__ unsigned page_valid_bits(int len, int pg) {
  const int nvalid = min(kPage, len - pg * kPage);
  return nvalid >= kPage ? 0xFFFFu : (nvalid <= 0 ? 0u : ((1u << nvalid) - 1u));
}

__global__ __launch_bounds__(kChunkPages) void plan_kernel(
    Dev d, const uint8_t *__restrict__ mask, const int32_t *__restrict__ new_pos,
    const int32_t *__restrict__ old_pos, int mode, int max_groups) {
  __shared__ int s_wave[kChunkPages / 64 + 1];
  __shared__ int s_last, s_gerr, s_fdrop, s_ok, s_nextra;
  __shared__ int s_src[kChunkPages * kPage], s_dlt[kChunkPages * kPage];
  __shared__ int s_lsrc[kChunkPages * kPage];
  const int c = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const size_t S = (size_t)d.S;
  const int len = ((mode & M_FORK) && d.fork_dst[b] < 0) ? 0 : d.lens[b];
  const int P = (len + kPage - 1) / kPage;
  const int pg = c * kChunkPages + t;
  if (c * kChunkPages < P) {
    // all loads of this thread's page first
    const int32_t *trow = d.table + (size_t)b * d.maxpg;
    unsigned keep = page_valid_bits(len, pg);
    uint4 m = make_uint4(0, 0, 0, 0);
    int tb = 0;
    int4 pp[4], oo[4];
    if (keep) {
      if (mode & M_DROP) m = *reinterpret_cast<const uint4 *>(mask + b * S + (size_t)pg * kPage);
      tb = trow[pg];
      if (mode & M_REPOS) {
        const int4 *ps = reinterpret_cast<const int4 *>(d.pos + (size_t)tb * kPage);
#pragma unroll
        for (int k = 0; k < 4; ++k) pp[k] = ps[k];
        if (mode & M_OLDPOS) {
          const int4 *os = reinterpret_cast<const int4 *>(old_pos + b * S + (size_t)pg * kPage);
#pragma unroll
          for (int k = 0; k < 4; ++k) oo[k] = os[k];
        }
      }
    }
    // survivor rank of the chunk's first page: the keep bits of the
    // sequence's earlier chunks, recounted (one page per thread per chunk;
    // eight chunks' mask words are loaded before any is counted, so the
    // loads overlap instead of costing one round trip per chunk)
    int acc = 0;
    for (int cc0 = 0; cc0 < c; cc0 += 8) {
      unsigned kq[8];
      uint4 mq[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int pq = (cc0 + u) * kChunkPages + t;
        kq[u] = cc0 + u < c ? page_valid_bits(len, pq) : 0u;
        mq[u] = (kq[u] && (mode & M_DROP))
                    ? *reinterpret_cast<const uint4 *>(mask + b * S + (size_t)pq * kPage)
                    : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += __popc(kq[u] & ~page_drop_bits(mq[u]));
    }
    if (t == 0) s_fdrop = INT_MAX;
    int base;
    block_exclusive_scan<kChunkPages>(acc, s_wave, &base);
    if (keep && (mode & M_DROP)) {
      const unsigned dropbits = page_drop_bits(m) & keep;
      keep &= ~dropbits;
      if (dropbits) atomicMin(&s_fdrop, pg * kPage + __ffs(dropbits) - 1);
    }
    int total;
    const int excl = block_exclusive_scan<kChunkPages>(__popc(keep), s_wave, &total);
    if (t == 0) {
      int *ci = d.chunk_info + ((size_t)b * d.nchunk + c) * 2;
      ci[0] = total;
      ci[1] = s_fdrop;
    }
    int err = 0, fpos = INT_MAX;
    if (keep) {
      const int j0 = base + excl;
      int p[kPage], o[kPage], qn[kPage];
      int qprev = -1;
      if (mode & M_REPOS) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          p[4 * k] = pp[k].x; p[4 * k + 1] = pp[k].y; p[4 * k + 2] = pp[k].z; p[4 * k + 3] = pp[k].w;
          if (mode & M_OLDPOS) {
            o[4 * k] = oo[k].x; o[4 * k + 1] = oo[k].y; o[4 * k + 2] = oo[k].z; o[4 * k + 3] = oo[k].w;
          }
        }
        if (mode & M_NEWPOS) {
          // slot r's survivor rank is j0 + (kept slots below r)
#pragma unroll
          for (int r = 0; r < kPage; ++r)
            qn[r] = ((keep >> r) & 1u) ? new_pos[b * S + j0 + __popc(keep & ((1u << r) - 1u))] : 0;
          if (j0 > 0) qprev = new_pos[b * S + j0 - 1];
        }
      }
      int j = j0;
#pragma unroll
      for (int r = 0; r < kPage; ++r) {
        if (!((keep >> r) & 1u)) continue;
        s_lsrc[j - base] = pg * kPage + r;                                 // pre-op index
        if (mode & (M_DROP | M_FORK)) s_src[j - base] = tb * kPage + r;   // physical slot
        if (mode & M_REPOS) {
          if ((mode & M_OLDPOS) && o[r] != p[r]) err = max(err, (int)AKV_ERR_POS_MISMATCH);
          int q = j;
          if (mode & M_NEWPOS) {
            q = qn[r];
            if (q < 0 || (j > 0 && qprev >= q)) err = max(err, (int)AKV_ERR_ORDER);
            qprev = q;
          }
          const int delta = q - p[r];
          s_dlt[j - base] = delta;
          if (delta != 0 && j < fpos) fpos = j;
        }
        ++j;
      }
    }
    __syncthreads();
    for (int i = t; i < total; i += kChunkPages) {
      if (mode & (M_DROP | M_FORK)) d.src_map[b * S + base + i] = s_src[i];
      if (mode & M_REPOS) d.delta_map[b * S + base + i] = s_dlt[i];
      d.last_src[b * S + base + i] = s_lsrc[i];
    }
    int *si = d.seq_info + (size_t)b * kSeqInfo;
    if (err) atomicMax(&si[SI_ERR], err);
    if (fpos != INT_MAX) atomicMin(&si[SI_FPOS], fpos);
  }
  // ---- last workgroup: finalize every sequence, prefix sums, pool check ----
  // Two-level ticket: chunks past a sequence's pages have nothing to report
  // and leave at once; the chunks of a sequence count on its own ticket, and
  // the last of them takes the one global ticket for the sequence, so the
  // global counter sees B increments instead of one per workgroup (1024 on
  // the 64-sequence batch, where contention on it cost ~100 us).
  if (gridDim.x * gridDim.y > 1) {
    const int nch_b = max(1, (P + kChunkPages - 1) / kChunkPages);
    if (c >= nch_b) return;
#if AKV_PLAN_SCOPED_FENCES
    // One thread orders the workgroup's records (every wave's stores precede
    // the barrier) before its ticket with a release fence, and the last
    // workgroup acquires them all: one L2 write-back and one invalidate on
    // the way to the finalize instead of full fences around each step.
    __syncthreads();
    if (t == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      bool seq_done = true;
      if (nch_b > 1) {
        int *tk = &d.seq_info[(size_t)b * kSeqInfo + SI_TICKET];
        seq_done = atomicAdd(tk, 1) == nch_b - 1;
        if (seq_done) *tk = 0;          // re-armed for the next op
        // the sequence's chunks, acquired, are released again with the global ticket
        if (seq_done && gridDim.y > 1) __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "agent");
      }
      // (one sequence: its own ticket already names the last workgroup)
      s_last = seq_done && (gridDim.y == 1 || atomicAdd(&d.ctl[CTL_DONE], 1) == (int)gridDim.y - 1);
      if (s_last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
    if (!s_last) return;
#else
    __threadfence();
    __syncthreads();
    if (t == 0) {
      bool seq_done = true;
      if (nch_b > 1) {
        int *tk = &d.seq_info[(size_t)b * kSeqInfo + SI_TICKET];
        seq_done = atomicAdd(tk, 1) == nch_b - 1;
        if (seq_done) *tk = 0;          // re-armed for the next op
        __threadfence();                // the sequence's chunks before the global ticket
      }
      // (one sequence: its own ticket already names the last workgroup)
      s_last = seq_done && (gridDim.y == 1 || atomicAdd(&d.ctl[CTL_DONE], 1) == (int)gridDim.y - 1);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
#endif
  } else {
    __syncthreads();
  }
  // the free count and the latched error, loaded now so that their round
  // trip overlaps the per-sequence pass below
  int fc_pre = 0, latched_pre = 0;
  if (t == 0) {
    s_gerr = 0;
    s_nextra = 0;
    fc_pre = *d.free_count;
    latched_pre = d.ctl[CTL_ERR];
  }
  __syncthreads();
  int run_m = 0, run_i = 0, run_f = 0;
  for (int b0 = 0; b0 < d.B; b0 += kChunkPages) {
    const int bb = b0 + t;
    int nm = 0, ni = 0, nf = 0, nfx = 0;
    int *si = d.seq_info + (size_t)bb * kSeqInfo;
    if (bb < d.B) {
      const int dst = (mode & M_FORK) ? d.fork_dst[bb] : -1;
      const int L0 = ((mode & M_FORK) && dst < 0) ? 0 : d.lens[bb];
      const int P0 = (L0 + kPage - 1) / kPage;
      const int nch = (P0 + kChunkPages - 1) / kChunkPages;
      int rnew = 0, fdrop = INT_MAX;
      for (int cc0 = 0; cc0 < nch; cc0 += 8) {
        int cn[8], cf[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int *ci = d.chunk_info + ((size_t)bb * d.nchunk + cc0 + u) * 2;
          cn[u] = cc0 + u < nch ? __atomic_load_n(&ci[0], __ATOMIC_RELAXED) : 0;
          cf[u] = cc0 + u < nch ? __atomic_load_n(&ci[1], __ATOMIC_RELAXED) : INT_MAX;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          rnew += cn[u];
          fdrop = min(fdrop, cf[u]);
        }
      }
      const int fpos = nch ? __atomic_load_n(&si[SI_FPOS], __ATOMIC_RELAXED) : INT_MAX;
      const int e = nch ? __atomic_load_n(&si[SI_ERR], __ATOMIC_RELAXED) : 0;
      // re-armed for the next op (the workgroups of a plan only lower / raise them)
      si[SI_FPOS] = INT_MAX;
      si[SI_ERR] = 0;
      const int Pn = (rnew + kPage - 1) / kPage;
      const int nsh = si[SI_NSHARED];   // pages [0, nsh) may be shared
      int fbd = P0;
      int ee = e;
      int sh_new = nsh;
      if (mode & M_FORK) {
        // The version shares the source's leading full pages whose entries it
        // leaves as they are (before the first dropped entry and the first
        // changed position; ranks equal indices there); every other survivor
        // goes to fresh pages of the (empty) destination.
        int keep_n = min(fdrop, L0);
        if ((mode & M_REPOS) && fpos < keep_n) keep_n = fpos;
        fbd = dst >= 0 ? keep_n / kPage : 0;
        nm = dst >= 0 ? Pn - fbd : 0;
        if (dst >= 0) sh_new = max(nsh, fbd);
        if (dst >= 0 && d.lens[dst] != 0) ee = max(ee, (int)AKV_ERR_ARG);
      } else if ((mode & M_DROP) && fdrop < L0) {
        fbd = fdrop / kPage;
        nm = max(0, Pn - fbd);
        nf = P0 - fbd;
      }
      int fip = P0;
      int nnext = (mode & M_FORK) && dst < 0 ? 0 : d.next_pos[bb];
      if (mode & M_REPOS) {
        if (fpos < rnew && !(mode & M_FORK)) {
          fip = fpos / kPage;
          ni = max(0, min(fbd, Pn) - fip);
          if (ni > 0 && fip < nsh) {
            // copy on write: a page another sequence may hold is never turned
            // in place; from the first changed page on, the sequence is
            // rebuilt in fresh pages
            fbd = fip;
            nm = max(0, Pn - fbd);
            nf = P0 - fbd;
            ni = 0;
          }
        }
        nnext = rnew == 0 ? 0 : ((mode & M_NEWPOS) ? new_pos[(size_t)bb * S + rnew - 1] + 1 : rnew);
      }
      // released pages [fbd, fbd + nf): the first ms may be held by other
      // sequences too (reference-counted), the rest return to the free stack
      int ms = 0;
      if (!(mode & M_FORK)) {
        ms = max(0, min(nsh, fbd + nf) - fbd);
        sh_new = min(nsh, fbd);
      }
      nfx = nf - ms;
      si[SI_NEW_LEN] = rnew;
      si[SI_FBD] = fbd;
      si[SI_FIP] = fip;
      si[SI_N_MOVE] = nm;
      si[SI_N_INPLACE] = ni;
      si[SI_N_FREED] = nf;
      si[SI_N_SHREL] = ms;
      si[SI_SH_NEW] = sh_new;
      si[SI_NEW_NEXT] = nnext;
      si[SI_OLD_LEN] = L0;
      si[SI_DST] = dst;
      if (ee) atomicMax(&s_gerr, ee);
    }
    int tm, ti, tf;
    const int em = block_exclusive_scan<kChunkPages>(nm, s_wave, &tm);
    const int ei = block_exclusive_scan<kChunkPages>(ni, s_wave, &ti);
    const int ef = block_exclusive_scan<kChunkPages>(nfx, s_wave, &tf);   // pages pushed
    if (bb < d.B) {
      si[SI_MOVE_OFF] = run_m + em;
      si[SI_INPLACE_OFF] = run_i + ei;
      si[SI_FREED_OFF] = run_f + ef;
    }
    run_m += tm;
    run_i += ti;
    run_f += tf;
  }
  __syncthreads();
  if (t == 0) {
    int e = s_gerr;
    const int fc = fc_pre;
    const int latched = latched_pre;
    int ng = 0;
    if (!e && !latched) {
      if (run_m <= fc) {
        int *gr = d.groups;
        gr[GR_S0] = 0; gr[GR_S1] = d.B; gr[GR_TM] = run_m; gr[GR_TI] = run_i; gr[GR_FC] = fc;
        gr[GR_MOFF] = 0; gr[GR_IOFF] = 0; gr[GR_FOFF] = 0; gr[GR_F] = run_f;
        ng = 1;
      } else if (max_groups > 1 && !(mode & M_FORK)) {
        // Too few free pages for the whole op: consecutive sequences are
        // grouped greedily, each group taking what is free when it starts
        // (the free count then grows by the pages the group drops).  Only a
        // sequence that does not fit on its own, or more groups than the
        // host launches rounds for, rejects the op.
        int fcur = fc, s0 = 0, gm = 0, gi = 0, gf = 0;
        auto close = [&](int s1) {
          const int *si0 = d.seq_info + (size_t)s0 * kSeqInfo;
          int *gr = d.groups + (size_t)ng * kGroupRec;
          gr[GR_S0] = s0; gr[GR_S1] = s1; gr[GR_TM] = gm; gr[GR_TI] = gi; gr[GR_FC] = fcur;
          gr[GR_MOFF] = si0[SI_MOVE_OFF]; gr[GR_IOFF] = si0[SI_INPLACE_OFF];
          gr[GR_FOFF] = si0[SI_FREED_OFF]; gr[GR_F] = gf;
          ++ng;
          fcur += gf - gm;
          s0 = s1;
          gm = gi = gf = 0;
        };
        for (int bb = 0; bb < d.B && !e; ++bb) {
          const int *si = d.seq_info + (size_t)bb * kSeqInfo;
          const int nm = si[SI_N_MOVE];
          if (gm + nm > fcur && bb > s0) {
            if (ng + 1 >= max_groups) e = AKV_ERR_NO_BLOCKS;
            else close(bb);
          }
          if (!e && nm > fcur) e = AKV_ERR_NO_BLOCKS;
          gm += nm;
          gi += si[SI_N_INPLACE];
          gf += si[SI_N_FREED] - si[SI_N_SHREL];
        }
        if (!e) close(d.B);
      } else {
        e = AKV_ERR_NO_BLOCKS;
      }
    }
    if (e || latched) {
      if (!latched) d.ctl[CTL_ERR] = e;
      d.ctl[CTL_OP_OK] = 0;
      d.ctl[CTL_NGROUPS] = 0;
      d.ctl[CTL_NPG0] = 0;
    } else {
      d.ctl[CTL_OP_OK] = 1;
      d.ctl[CTL_NGROUPS] = ng;
      d.ctl[CTL_MODE] = mode;
      d.ctl[CTL_NPG0] = d.groups[GR_TM] + d.groups[GR_TI];
    }
    d.ctl[CTL_DONE] = 0;
    s_ok = !(e || latched);
  }
  __syncthreads();
  // Gather map of this op for akv_query_state: sequence b's row of last_src
  // (a fork destination reads its source's row); none after a rejected op.
  for (int bb = t; bb < d.B; bb += kChunkPages) {
    int *si = d.seq_info + (size_t)bb * kSeqInfo;
    const bool own = s_ok && !(mode & M_FORK);
    si[SI_LSRC_ROW] = own ? bb : -1;
    si[SI_LSRC_LEN] = own ? si[SI_NEW_LEN] : 0;
  }
  __syncthreads();
  if (s_ok && (mode & M_FORK))
    for (int bb = t; bb < d.B; bb += kChunkPages) {
      const int dst = d.fork_dst[bb];
      if (dst >= 0) {
        int *sd = d.seq_info + (size_t)dst * kSeqInfo;
        sd[SI_LSRC_ROW] = bb;
        sd[SI_LSRC_LEN] = d.seq_info[(size_t)bb * kSeqInfo + SI_NEW_LEN];
      }
    }
  if (s_ok) {
    // shared prefixes: every planned sequence's bound after the op; a fork's
    // destination shares its source's first SI_FBD pages
    for (int bb = t; bb < d.B; bb += kChunkPages) {
      int *si = d.seq_info + (size_t)bb * kSeqInfo;
      if (!(mode & M_FORK) || d.fork_dst[bb] >= 0) si[SI_NSHARED] = si[SI_SH_NEW];
    }
    __syncthreads();
    if (mode & M_FORK) {
      for (int bb = t; bb < d.B; bb += kChunkPages) {
        const int dst = d.fork_dst[bb];
        if (dst >= 0)
          d.seq_info[(size_t)dst * kSeqInfo + SI_NSHARED] = d.seq_info[(size_t)bb * kSeqInfo + SI_FBD];
      }
    } else {
      // Released pages that may be shared lose one reference; a page whose
      // last reference this was goes on the list the op's last commit round
      // pushes (after every move has read its fresh page ids).  The list's
      // order follows the atomics; the pages are the same either way.
      for (int bb = t; bb < d.B; bb += kChunkPages) {
        const int *si = d.seq_info + (size_t)bb * kSeqInfo;
        const int ms = si[SI_N_SHREL];
        const int32_t *trow = d.table + (size_t)bb * d.maxpg + si[SI_FBD];
        for (int k0 = 0; k0 < ms; k0 += 8) {
          int pgs[8], old[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) pgs[u] = k0 + u < ms ? trow[k0 + u] : -1;
#pragma unroll
          for (int u = 0; u < 8; ++u) old[u] = pgs[u] >= 0 ? atomicSub(&d.share[pgs[u]], 1) : 1;
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (old[u] == 0) {
              d.share[pgs[u]] = 0;
              d.ex_list[atomicAdd(&s_nextra, 1)] = pgs[u];
            }
        }
      }
    }
    __syncthreads();
    if (t == 0) d.ctl[CTL_NEXTRA] = s_nextra;
  }
  if (s_ok && (mode & M_STAGED)) {
    // One-sequence cache (one group, no fork): commit here.  The fresh page
    // ids go to the staging array first (the move reads them there, not from
    // the free stack), then the old pages are pushed over the region they
    // came from, so nothing of the commit waits for the move; the move runs
    // after this kernel in stream order and reads only plan records, source
    // slots and the untouched prefix of the page table.
    // (each thread loads a batch of 8 before storing any: independent loads
    // in flight instead of one round trip per entry)
    constexpr int kB = 8;
    const int *gr = d.groups;
    const int Tm = gr[GR_TM], fc0 = gr[GR_FC], F = gr[GR_F];
    const int *si = d.seq_info;
    const int fbd = si[SI_FBD], nmove = si[SI_N_MOVE], nfreed = si[SI_N_FREED];
    const int base = fc0 - Tm;
    int32_t *trow = d.table;
    // (a one-sequence cache shares no page: every released page is pushed,
    // F == nfreed)
    if (Tm <= kChunkPages * kB && nfreed <= kChunkPages * kB) {
      // one pass: every entry read (fresh page ids from the top of the free
      // stack, the table entries they replace), one barrier, then the writes
      // -- the pushed pages land where the fresh ones were popped
      int fresh[kB], old[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const int k = t + u * kChunkPages;
        fresh[u] = k < Tm ? d.free_stack[fc0 - 1 - k] : -1;
        old[u] = k < nfreed ? trow[fbd + k] : 0;
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const int k = t + u * kChunkPages;
        if (k < Tm) d.stage[k] = fresh[u];
        if (k < nfreed) {
          d.free_stack[base + F - 1 - k] = old[u];   // reversed, as in commit_kernel
          trow[fbd + k] = k < nmove ? fresh[u] : -1;
        }
      }
      if (t == 0) {
        d.lens[0] = si[SI_NEW_LEN];
        d.next_pos[0] = si[SI_NEW_NEXT];
        *d.free_count = base + F;
      }
      return;
    }
    for (int k0 = t; k0 < Tm; k0 += kChunkPages * kB) {
      int v[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const int k = k0 + u * kChunkPages;
        v[u] = k < Tm ? d.free_stack[fc0 - 1 - k] : 0;
      }
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const int k = k0 + u * kChunkPages;
        if (k < Tm) d.stage[k] = v[u];
      }
    }
    __syncthreads();
    for (int k0 = t; k0 < nfreed; k0 += kChunkPages * kB) {
      int old[kB], fresh[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const int k = k0 + u * kChunkPages;
        old[u] = k < nfreed ? trow[fbd + k] : 0;
        fresh[u] = k < nmove ? d.stage[k] : -1;
      }
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const int k = k0 + u * kChunkPages;
        if (k < nfreed) {
          d.free_stack[base + F - 1 - k] = old[u];   // reversed, as in commit_kernel
          trow[fbd + k] = fresh[u];
        }
      }
    }
    if (t == 0) {
      d.lens[0] = si[SI_NEW_LEN];
      d.next_pos[0] = si[SI_NEW_NEXT];
      *d.free_count = base + F;
    }
  }
}

// ---------------------------------------------------------------------------
// commit
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void commit_kernel(Dev d, int group) {
  const int ng = d.ctl[CTL_NGROUPS];
  if (d.ctl[CTL_OP_OK] == 0 || group >= ng) return;
  const int *gr = d.groups + (size_t)group * kGroupRec;
  const int b = blockIdx.x;
  const int s0 = gr[GR_S0];
  if (b < s0 || b >= gr[GR_S1]) return;
  const int *si = d.seq_info + (size_t)b * kSeqInfo;
  const int fbd = si[SI_FBD], nmove = si[SI_N_MOVE], nfreed = si[SI_N_FREED];
  const int ms = si[SI_N_SHREL];
  const int moff = si[SI_MOVE_OFF], foff = si[SI_FREED_OFF] - gr[GR_FOFF];
  const int base = gr[GR_FC] - gr[GR_TM];   // the group's fresh pages came from [base, GR_FC)
  const int ftot = gr[GR_F];
  // The op's last round also pushes the shared pages the plan saw released
  // for the last time, above the group's own.
  const int nx = (group == ng - 1) ? d.ctl[CTL_NEXTRA] : 0;
  if (b == s0) {
    for (int i = threadIdx.x; i < nx; i += blockDim.x) d.free_stack[base + ftot + i] = d.ex_list[i];
    if (threadIdx.x == 0) *d.free_count = base + ftot + nx;
  }
  const int dst = si[SI_DST];
  if (dst >= 0) {
    // fork: the new version holds the source's first fbd pages too (one more
    // reference each) and takes the fresh pages after them; the source's
    // page table is untouched
    const int32_t *srow = d.table + (size_t)b * d.maxpg;
    int32_t *drow = d.table + (size_t)dst * d.maxpg;
    for (int k = threadIdx.x; k < fbd; k += blockDim.x) {
      const int pg = srow[k];
      drow[k] = pg;
      atomicAdd(&d.share[pg], 1);
    }
    for (int k = threadIdx.x; k < nmove; k += blockDim.x) drow[fbd + k] = d.stage[moff + k];
    if (threadIdx.x == 0) {
      d.lens[dst] = si[SI_NEW_LEN];
      d.next_pos[dst] = si[SI_NEW_NEXT];
    }
    return;
  }
  if (d.ctl[CTL_MODE] & M_FORK) return;
  // The freed pages go onto the stack in reverse (sequence b's first page on
  // top of b + 1's), so later pops hand them out in their old order: a
  // sequence rebuilt from them keeps ascending page runs, and the move's
  // blocks in flight keep reading and writing compact address ranges (a
  // scattered page table costs the move ~11% on MI355X).  The first ms
  // released pages may be held by other sequences: the plan has already
  // counted their references down.
  int32_t *trow = d.table + (size_t)b * d.maxpg;
  for (int k = threadIdx.x; k < nfreed; k += blockDim.x) {
    const int po = fbd + k;
    const int old = trow[po];
    if (k >= ms) d.free_stack[base + ftot - 1 - (foff + k - ms)] = old;
    trow[po] = (k < nmove) ? d.stage[moff + k] : -1;
  }
  if (threadIdx.x == 0) {
    d.lens[b] = si[SI_NEW_LEN];
    d.next_pos[b] = si[SI_NEW_NEXT];
  }
}

// akv_fork's destination map, carried in the kernel's arguments (copied by
// the runtime at launch, so the caller's host array may go away at once).
constexpr int kForkMapChunk = 512;
struct ForkMapChunk {
  int32_t v[kForkMapChunk];
};
__global__ __launch_bounds__(kForkMapChunk) void fork_map_kernel(Dev d, int off, int n,
                                                                 ForkMapChunk m) {
  const int i = threadIdx.x;
  if (i < n) d.fork_dst[off + i] = m.v[i];
}

// ---------------------------------------------------------------------------
// append ([CE] eq. 3)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kPlanThreads) void append_plan_kernel(Dev d, const int32_t *counts) {
  __shared__ int s_wave[kPlanThreads / 64 + 1];
  __shared__ int s_err;
  const int t = threadIdx.x;
  if (t == 0) s_err = 0;
  __syncthreads();
  int run_n = 0, run_p = 0;
  for (int base = 0; base < d.B; base += kPlanThreads) {
    const int b = base + t;
    int n = 0, need = 0;
    if (b < d.B) {
      n = counts[b];
      const int old = d.lens[b];
      const int po = (old + kPage - 1) / kPage;
      const long long pn = ((long long)old + n + kPage - 1) / kPage;
      if (n < 0) atomicMax(&s_err, (int)AKV_ERR_ARG);
      else if (pn > d.maxpg) atomicMax(&s_err, (int)AKV_ERR_CAPACITY);
      else need = (int)pn - po;
      int *si = d.seq_info + (size_t)b * kSeqInfo;
      si[SI_OLD_LEN] = old;
      si[SI_OLD_NEXT] = d.next_pos[b];
      si[SI_N_MOVE] = need;
    }
    int tn, tp;
    const int en = block_exclusive_scan<kPlanThreads>(max(n, 0), s_wave, &tn);
    const int ep = block_exclusive_scan<kPlanThreads>(need, s_wave, &tp);
    if (b < d.B) {
      int *si = d.seq_info + (size_t)b * kSeqInfo;
      si[SI_APP_OFF] = run_n + en;
      si[SI_MOVE_OFF] = run_p + ep;
    }
    run_n += tn;
    run_p += tp;
  }
  __syncthreads();
  const int fc = *d.free_count;
  __shared__ int s_ok;
  if (t == 0) {
    int e = s_err;
    if (!e && run_p > fc) e = AKV_ERR_NO_BLOCKS;
    const int latched = d.ctl[CTL_ERR];
    if (e && !latched) d.ctl[CTL_ERR] = e;
    s_ok = !(e || latched);
    d.ctl[CTL_OP_OK] = s_ok;
  }
  __syncthreads();
  if (!s_ok) return;
  for (int b = 0; b < d.B; ++b) {
    const int *si = d.seq_info + (size_t)b * kSeqInfo;
    const int need = si[SI_N_MOVE], off = si[SI_MOVE_OFF];
    const int po = (si[SI_OLD_LEN] + kPage - 1) / kPage;
    for (int k = t; k < need; k += kPlanThreads)
      d.table[(size_t)b * d.maxpg + po + k] = d.free_stack[fc - 1 - (off + k)];
  }
  __syncthreads();
  for (int base = 0; base < d.B; base += kPlanThreads) {
    const int b = base + t;
    if (b < d.B) {
      const int n = counts[b];
      const int *si = d.seq_info + (size_t)b * kSeqInfo;
      d.lens[b] = si[SI_OLD_LEN] + n;
      d.next_pos[b] = si[SI_OLD_NEXT] + n;
    }
  }
  if (t == 0) *d.free_count = fc - run_p;
}

// Append copy.  One workgroup per (layer group, 16 new tokens), in
// layer-major order (the token group varies fastest), so the workgroups in
// flight read a compact range of the input and write a compact range of the
// pages.  16 lanes find their token's page, row and position (positions and
// token ids are written by the first layer group); the workgroup then copies
// its tokens' K/V rows of every kv head with 16-B accesses, a batch of loads
// issued before their stores.  With ROPE the keys arrive unrotated and are
// turned to each token's position p on the way (the model's RoPE step fused
// into the append): cos/sin of p * theta_i in fp64 per token in LDS, each
// rotary chunk pair rotated in fp64 and rounded once, the non-rotary tail
// copied.
#ifndef AKV_APPEND_BATCH
#define AKV_APPEND_BATCH 2       // plain append: 16-B chunks per plane loaded before they are stored
#endif
#ifndef AKV_APPEND_ROPE_BATCH
#define AKV_APPEND_ROPE_BATCH 8  // the same for the RoPE-fused append
#endif
// (Llama-8B shape, 32768 tokens, two A/B pairs on one box: plain batch 2
// 0.694-0.697 of the HBM peak vs 4 0.685, 1 0.690, 8 0.674; RoPE-fused
// batch 8 0.718 vs 4 0.711-0.715)
constexpr int append_batch(bool rope) { return rope ? AKV_APPEND_ROPE_BATCH : AKV_APPEND_BATCH; }
constexpr int kAppTok = 16;                      // new tokens per workgroup
#ifndef AKV_APPEND_LAYERS
#define AKV_APPEND_LAYERS 2
#endif
#ifndef AKV_APPEND_ROPE_LAYERS
#define AKV_APPEND_ROPE_LAYERS 1
#endif
// layers per workgroup (measured on 32768 tokens at the Llama-8B shape:
// plain 2 layers 5.47 TB/s vs 1 layer 5.42; RoPE-fused 1 layer 5.68 vs 2
// layers 5.51 and 4 layers 5.36 -- the per-token cos/sin are cheap to redo)
constexpr int append_layers(bool rope) { return rope ? AKV_APPEND_ROPE_LAYERS : AKV_APPEND_LAYERS; }

// Inputs are read once and the pages written once: streamed with the
// nontemporal hint where every access instruction covers whole 128-B lines.
template <bool NT>
__device__ __forceinline__ u32x4 ld_once(const uint16_t *p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  else return *reinterpret_cast<const u32x4 *>(p);
}
template <bool NT>
__device__ __forceinline__ void st_once(uint16_t *p, u32x4 v) {
  if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
  else *reinterpret_cast<u32x4 *>(p) = v;
}

template <int D, bool ROPE>
__global__ __launch_bounds__(256) void append_copy_kernel(Dev d, int64_t n_new, int ntg,
                                                          const uint16_t *__restrict__ k_new,
                                                          const uint16_t *__restrict__ v_new,
                                                          const int32_t *__restrict__ tok_new) {
  if (d.ctl[CTL_OP_OK] == 0) return;
  constexpr int LPB = append_layers(ROPE);
  constexpr int kAppendBatch = append_batch(ROPE);
  constexpr int C8 = D / 8;                    // 16-B chunks per row
  __shared__ int s_page[kAppTok], s_row[kAppTok], s_pos[kAppTok];
  __shared__ double2 s_cs[ROPE ? kAppTok : 1][ROPE ? kMaxHalf : 1];
  const int tg = blockIdx.x % ntg, lg = blockIdx.x / ntg;
  const int64_t tk0 = (int64_t)tg * kAppTok;
  const int ntok = (int)min<int64_t>(kAppTok, n_new - tk0);
  const int t = threadIdx.x;
  if (t < ntok) {
    const int64_t tk = tk0 + t;
    int lo = 0, hi = d.B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (d.seq_info[(size_t)mid * kSeqInfo + SI_APP_OFF] <= tk) lo = mid; else hi = mid - 1;
    }
    // sequences that append nothing share the offset of the next one: the
    // search lands on the last sequence whose offset is <= tk
    const int *si = d.seq_info + (size_t)lo * kSeqInfo;
    const int j = (int)(tk - si[SI_APP_OFF]);
    const int slot = si[SI_OLD_LEN] + j;
    const int page = d.table[(size_t)lo * d.maxpg + slot / kPage];
    s_page[t] = page;
    s_row[t] = slot % kPage;
    s_pos[t] = si[SI_OLD_NEXT] + j;
    if (lg == 0) {
      d.pos[(size_t)page * kPage + slot % kPage] = si[SI_OLD_NEXT] + j;
      d.tok[(size_t)page * kPage + slot % kPage] = tok_new[tk];
    }
  }
  if constexpr (ROPE) {
    __syncthreads();
    const int RH = d.RD / 2;
    for (int task = t; task < ntok * RH; task += blockDim.x) {
      const int i = task / RH, pr = task - i * RH;
      const int pos = s_pos[i];
      double sn = 0.0, cs = 1.0;
      if (pos != 0) sincos_rope((double)pos * d.theta[pr], &sn, &cs);
      s_cs[i][pr] = make_double2(cs, sn);
    }
  }
  __syncthreads();
  const PoolStrides ps = pool_strides(d.NB, d.H, D);
  const int l_lo = lg * LPB, l_hi = min(d.L, l_lo + LPB);
  for (int l = l_lo; l < l_hi; ++l) {
    if constexpr (ROPE) {
      constexpr int CH = D / 16;               // chunk pairs per row
      // a chunk pair's x and y halves are whole 128-B lines only at d = 128
      constexpr bool NTP = D == 128;
      const int rch = d.RD / 16;
      const int npair = ntok * d.H * CH;
      for (int c0 = t; c0 < npair; c0 += blockDim.x * kAppendBatch) {
        u32x4 x[kAppendBatch], y[kAppendBatch];
        size_t dst[kAppendBatch];
        int yo[kAppendBatch], pcs[kAppendBatch], tix[kAppendBatch];
#pragma unroll
        for (int u = 0; u < kAppendBatch; ++u) {
          const int c = c0 + u * blockDim.x;
          if (c >= npair) continue;
          const int pc = c % CH, ih = c / CH, h = ih % d.H, i = ih / d.H;
          const bool rot = pc < rch;
          const int xo = rot ? 8 * pc : d.RD + 8 * (pc - rch);
          yo[u] = rot ? d.RD / 2 : (D - d.RD) / 2;
          pcs[u] = pc;
          tix[u] = i;
          const size_t src = (((size_t)l * n_new + tk0 + i) * d.H + h) * D + xo;
          dst[u] = (size_t)l * ps.layer + (size_t)s_page[i] * ps.page + (size_t)h * ps.head +
                   (size_t)s_row[i] * D + xo;
          x[u] = ld_once<NTP>(k_new + src);
          y[u] = ld_once<NTP>(k_new + src + yo[u]);
        }
#pragma unroll
        for (int u = 0; u < kAppendBatch; ++u) {
          if (c0 + u * (int)blockDim.x >= npair) continue;
          if (pcs[u] < rch && s_pos[tix[u]] != 0) rotate8(x[u], y[u], &s_cs[tix[u]][8 * pcs[u]]);
          st_once<NTP>(d.k + dst[u], x[u]);
          st_once<NTP>(d.k + dst[u] + yo[u], y[u]);
        }
      }
    }
    const int nchunk = ntok * d.H * C8;
    for (int c0 = t; c0 < nchunk; c0 += blockDim.x * kAppendBatch) {
      u32x4 kk[kAppendBatch], vv[kAppendBatch];
      size_t dst[kAppendBatch];
#pragma unroll
      for (int u = 0; u < kAppendBatch; ++u) {
        const int c = c0 + u * blockDim.x;
        if (c >= nchunk) continue;
        const int e8 = c % C8, ih = c / C8, h = ih % d.H, i = ih / d.H;
        const size_t src = (((size_t)l * n_new + tk0 + i) * d.H + h) * D + 8 * e8;
        dst[u] = (size_t)l * ps.layer + (size_t)s_page[i] * ps.page + (size_t)h * ps.head +
                 (size_t)s_row[i] * D + 8 * e8;
        if constexpr (!ROPE) kk[u] = ld_once<true>(k_new + src);
        vv[u] = ld_once<true>(v_new + src);
      }
#pragma unroll
      for (int u = 0; u < kAppendBatch; ++u) {
        if (c0 + u * (int)blockDim.x >= nchunk) continue;
        if constexpr (!ROPE) st_once<true>(d.k + dst[u], kk[u]);
        st_once<true>(d.v + dst[u], vv[u]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// release: the flagged sequences' pages go back on the free stack
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kPlanThreads) void release_kernel(Dev d, const uint8_t *sel) {
  __shared__ int s_wave[kPlanThreads / 64 + 1];
  __shared__ int s_ok, s_nx;
  __shared__ int s_np[kPlanThreads], s_ms[kPlanThreads], s_off[kPlanThreads];
  const int t = threadIdx.x;
  if (t == 0) {
    s_ok = d.ctl[CTL_ERR] == 0;    // a latched error makes mutating calls no-ops
    s_nx = 0;
  }
  __syncthreads();
  if (!s_ok) return;
  const int fc = *d.free_count;
  // pages a flagged sequence holds alone (at or past its shared bound) are
  // pushed in reverse (the first sequence's first page on top: later pops
  // return them in their old order); `all` counts them
  int all = 0;
  for (int base = 0; base < d.B; base += kPlanThreads) {
    const int b = base + t;
    int nx = 0;
    if (b < d.B && sel[b]) {
      const int np = (d.lens[b] + kPage - 1) / kPage;
      nx = np - min(np, d.seq_info[(size_t)b * kSeqInfo + SI_NSHARED]);
    }
    int tot;
    block_exclusive_scan<kPlanThreads>(nx, s_wave, &tot);
    all += tot;
  }
  int run = 0;
  for (int base = 0; base < d.B; base += kPlanThreads) {
    const int b = base + t;
    int np = 0, msb = 0;
    if (b < d.B && sel[b]) {
      np = (d.lens[b] + kPage - 1) / kPage;
      msb = min(np, d.seq_info[(size_t)b * kSeqInfo + SI_NSHARED]);
    }
    int tot;
    const int ex = block_exclusive_scan<kPlanThreads>(np - msb, s_wave, &tot);
    s_np[t] = np;
    s_ms[t] = msb;
    s_off[t] = run + ex;
    __syncthreads();
    // all threads walk this chunk's flagged sequences, one page each
    const int nb = min(kPlanThreads, d.B - base);
    for (int i = 0; i < nb; ++i) {
      const int n = s_np[i];
      if (n == 0) continue;
      const int m = s_ms[i], off = s_off[i];
      int32_t *row = d.table + (size_t)(base + i) * d.maxpg;
      for (int k = t; k < n; k += kPlanThreads) {
        const int pg = row[k];
        if (k >= m) {
          d.free_stack[fc + all - 1 - (off + k - m)] = pg;
        } else if (atomicSub(&d.share[pg], 1) == 0) {
          // the last reference to a shared page
          d.share[pg] = 0;
          d.ex_list[atomicAdd(&s_nx, 1)] = pg;
        }
        row[k] = -1;
      }
    }
    if (np || (b < d.B && sel[b])) {
      d.lens[b] = 0;
      d.next_pos[b] = 0;
      d.seq_info[(size_t)b * kSeqInfo + SI_NSHARED] = 0;
    }
    run += tot;
    __syncthreads();
  }
  for (int i = t; i < s_nx; i += kPlanThreads) d.free_stack[fc + all + i] = d.ex_list[i];
  if (t == 0) *d.free_count = fc + all + s_nx;
}

// ---------------------------------------------------------------------------
// reset
// ---------------------------------------------------------------------------
__global__ void reset_kernel(Dev d, const int32_t *order) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t ntab = (int64_t)d.B * d.maxpg;
  if (i < ntab) d.table[i] = -1;
  if (i < d.B) {
    d.lens[i] = 0;
    d.next_pos[i] = 0;
    d.seq_info[i * kSeqInfo + SI_FPOS] = INT_MAX;   // plan accumulators, re-armed by every plan
    d.seq_info[i * kSeqInfo + SI_ERR] = 0;
    d.seq_info[i * kSeqInfo + SI_LSRC_ROW] = -1;     // no gather map yet
    d.seq_info[i * kSeqInfo + SI_LSRC_LEN] = 0;
    d.seq_info[i * kSeqInfo + SI_NSHARED] = 0;      // nothing shared
    d.seq_info[i * kSeqInfo + SI_TICKET] = 0;
  }
  if (i < d.NB) {
    d.free_stack[d.NB - 1 - i] = order ? order[i] : (int)i;
    d.share[i] = 0;
  }
  if (i == 0) {
    *d.free_count = d.NB;
    for (int c = 0; c < CTL_COUNT; ++c) d.ctl[c] = 0;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_plan(const Dev &d, const uint8_t *mask, const int32_t *new_pos,
                       const int32_t *old_pos, int mode, int max_groups, hipStream_t st) {
  const dim3 grid(d.nchunk, d.B);
  hipLaunchKernelGGL(plan_kernel, grid, dim3(kChunkPages), 0, st, d, mask, new_pos, old_pos, mode,
                     max_groups);
  return hipGetLastError();
}

hipError_t launch_commit(const Dev &d, int group, hipStream_t st) {
  hipLaunchKernelGGL(commit_kernel, dim3(d.B), dim3(256), 0, st, d, group);
  return hipGetLastError();
}

hipError_t launch_fork_map(const Dev &d, const int32_t *dst_of_host, hipStream_t st) {
  for (int off = 0; off < d.B; off += kForkMapChunk) {
    ForkMapChunk m;
    const int n = std::min(kForkMapChunk, d.B - off);
    for (int i = 0; i < n; ++i) m.v[i] = dst_of_host[off + i];
    hipLaunchKernelGGL(fork_map_kernel, dim3(1), dim3(kForkMapChunk), 0, st, d, off, n, m);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_append(const Dev &d, const int32_t *counts, int64_t n_new,
                         const uint16_t *k_new, const uint16_t *v_new, const int32_t *tok_new,
                         bool rope, hipStream_t st) {
  hipLaunchKernelGGL(append_plan_kernel, dim3(1), dim3(kPlanThreads), 0, st, d, counts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_new == 0) return e;
  const int ntg = (int)((n_new + kAppTok - 1) / kAppTok);
  const int lpb = append_layers(rope);
  const dim3 g((unsigned)((long long)ntg * ((d.L + lpb - 1) / lpb))), b(256);
  if (d.D == 128) {
    if (rope) hipLaunchKernelGGL((append_copy_kernel<128, true>), g, b, 0, st, d, n_new, ntg, k_new, v_new, tok_new);
    else hipLaunchKernelGGL((append_copy_kernel<128, false>), g, b, 0, st, d, n_new, ntg, k_new, v_new, tok_new);
  } else {
    if (rope) hipLaunchKernelGGL((append_copy_kernel<64, true>), g, b, 0, st, d, n_new, ntg, k_new, v_new, tok_new);
    else hipLaunchKernelGGL((append_copy_kernel<64, false>), g, b, 0, st, d, n_new, ntg, k_new, v_new, tok_new);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// state export: lengths, next positions, and every sequence's positions and
// token ids in active order (slots past the length read -1)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void query_kernel(Dev d, int32_t *lens, int32_t *next,
                                                     int32_t *pos, int32_t *tok,
                                                     int32_t *last_src) {
  const int b = blockIdx.y;
  const int len = d.lens[b];
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (lens) lens[b] = len;
    if (next) next[b] = d.next_pos[b];
  }
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= d.S) return;
  if (pos || tok) {
    int p = -1, t = -1;
    if (j < len) {
      const size_t slot = (size_t)d.table[(size_t)b * d.maxpg + j / kPage] * kPage + j % kPage;
      p = d.pos[slot];
      t = d.tok[slot];
    }
    if (pos) pos[(size_t)b * d.S + j] = p;
    if (tok) tok[(size_t)b * d.S + j] = t;
  }
  if (last_src) {
    const int *si = d.seq_info + (size_t)b * kSeqInfo;
    const int row = si[SI_LSRC_ROW];
    last_src[(size_t)b * d.S + j] =
        (row >= 0 && j < si[SI_LSRC_LEN]) ? d.last_src[(size_t)row * d.S + j] : -1;
  }
}

hipError_t launch_query(const Dev &d, int32_t *lens, int32_t *next, int32_t *pos, int32_t *tok,
                        int32_t *last_src, hipStream_t st) {
  hipLaunchKernelGGL(query_kernel, dim3((unsigned)((d.S + 255) / 256), (unsigned)d.B), dim3(256),
                     0, st, d, lens, next, pos, tok, last_src);
  return hipGetLastError();
}

hipError_t launch_release(const Dev &d, const uint8_t *sel, hipStream_t st) {
  hipLaunchKernelGGL(release_kernel, dim3(1), dim3(kPlanThreads), 0, st, d, sel);
  return hipGetLastError();
}

hipError_t launch_reset(const Dev &d, const int32_t *order_dev, hipStream_t st) {
  const int64_t n = std::max<int64_t>((int64_t)d.B * d.maxpg, std::max<int64_t>(d.NB, d.B));
  const unsigned grid = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(reset_kernel, dim3(grid), dim3(256), 0, st, d, order_dev);
  return hipGetLastError();
}

}  // namespace akv
