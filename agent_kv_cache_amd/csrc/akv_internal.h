// Internal declarations shared by the libakv host code and kernels.
// Not part of the public ABI (see include/akv.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/akv.h"

namespace akv {

constexpr int kPage = 16;       // tokens per page
constexpr int kMaxHalf = 64;    // head_dim / 2 upper bound (head_dim <= 128)

// Control words at the start of the scratch buffer (int32 each).
enum Ctl : int {
  CTL_ERR = 0,        // latched error code (sticky until akv_sync_status)
  CTL_DONE = 1,       // last-block ticket of the plan kernels
  CTL_OP_OK = 2,      // 1 when the planned op may commit
  CTL_NGROUPS = 3,    // sequence groups of the planned op (move + commit rounds that run)
  CTL_NEXTRA = 4,     // shared pages the op released for the last time (pushed by the last round)
  CTL_NPG0 = 5,       // pages group 0 of the planned op rebuilds (0: nothing to move)
  CTL_MODE = 8,       // mode bits of the planned op
  CTL_COUNT = 64
};

// A drop / reposition whose new pages do not fit the free pool at once runs
// in groups of consecutive sequences, one (move, commit) round per group in
// stream order; a group's commit returns its old pages before the next group
// takes fresh ones.  Group record (int32 x kGroupRec), filled by the plan:
enum GroupRec : int {
  GR_S0 = 0,       // first sequence of the group
  GR_S1 = 1,       // one past its last sequence
  GR_TM = 2,       // pages moved out of place
  GR_TI = 3,       // pages re-rotated in place
  GR_FC = 4,       // free_count when the group starts
  GR_MOFF = 5,     // global move offset of its first moved page (SI_MOVE_OFF)
  GR_IOFF = 6,     // global in-place offset (SI_INPLACE_OFF)
  GR_FOFF = 7,     // global freed offset (SI_FREED_OFF)
  GR_F = 8,        // pages it returns to the free stack
  kGroupRec = 16
};
constexpr int kMaxOpGroups = 64;       // capacity of the group table
#ifndef AKV_MAX_OP_GROUPS
#define AKV_MAX_OP_GROUPS 8            // default rounds when the pool may run short
#endif

// Per-sequence plan record (int32 x kSeqInfo).
enum SeqInfo : int {
  SI_NEW_LEN = 0,    // survivors r'
  SI_FBD = 1,        // first page rewritten out of place (== pages if none)
  SI_FIP = 2,        // first page re-rotated in place
  SI_N_MOVE = 3,
  SI_N_INPLACE = 4,
  SI_N_FREED = 5,
  SI_NEW_NEXT = 6,   // next_pos after the op
  SI_ERR = 7,
  SI_MOVE_OFF = 8,   // exclusive prefix over sequences
  SI_INPLACE_OFF = 9,
  SI_FREED_OFF = 10,
  SI_OLD_LEN = 11,
  SI_OLD_NEXT = 12,
  SI_APP_OFF = 13,   // append: offset of this sequence's tokens in the input
  SI_FPOS = 14,      // first survivor rank whose position changes (atomic min)
  SI_DST = 15,       // fork: destination sequence (-1 = none)
  SI_LSRC_ROW = 16,  // row of last_src holding this sequence's gather map (-1: none)
  SI_LSRC_LEN = 17,  // entries of that map
  SI_NSHARED = 18,   // pages [0, NSHARED) of this sequence may be shared with other
                     // sequences (kept across ops; pages at or past it are its own)
  SI_N_SHREL = 19,   // the first N_SHREL released pages may be shared (reference-counted)
  SI_SH_NEW = 20,    // SI_NSHARED after the planned op
  SI_TICKET = 21,    // plan chunks of this sequence done (re-armed to 0 by the last)
  kSeqInfo = 24
};

// Ops that need at most this many one-shot blocks (one per layer group of
// each rebuilt page) are moved by a one-shot grid, larger ones by a
// persistent grid.
#ifndef AKV_MOVE_ONESHOT_CAP
#define AKV_MOVE_ONESHOT_CAP 131072
#endif
// Layers per one-shot block (0: 1 at head_dim 128, 2 at 64).  One layer at
// both sizes: at d = 64 a block then moves 32 KiB instead of 64, and the
// launch's tail is shorter (50-turn history, three alternating process pairs
// on one box: move 10.01-10.04 -> 9.91-9.94 ms).
#ifndef AKV_MOVE_OS_LAYERS
#define AKV_MOVE_OS_LAYERS 1
#endif

// Mode bits of the compaction plan.
enum Mode : int {
  M_DROP = 1,        // a drop mask is given
  M_REPOS = 2,       // positions change (canonical unless M_NEWPOS)
  M_NEWPOS = 4,      // explicit new positions
  M_OLDPOS = 8,      // validate old positions
  M_FORK = 16,       // write a new position version into an empty sequence
  M_STAGED = 32,     // one-sequence cache: the plan fills the fresh page ids into the
                     // staging array and commits the op itself (no commit kernel)
};

// Device view of one cache, passed by value to every kernel.
struct Dev {
  uint16_t *k, *v;
  int32_t *table, *lens, *next_pos, *pos, *tok, *free_stack, *free_count;
  int32_t *ctl, *seq_info, *src_map, *delta_map, *stage, *chunk_info, *fork_dst;
  int32_t *last_src;          // [B][S] gather map of the last drop / reposition / fork
  int32_t *share;             // [NB] references to a page beyond the first (0: one holder)
  int32_t *ex_list;           // [NB] shared pages an op released for the last time
  int32_t *groups;            // [kMaxOpGroups][kGroupRec] sequence groups of the planned op
  const double *theta;        // [RD/2] rotation frequencies
  const int32_t *window;      // [L] sliding-window length per layer, 0 = full attention
  int L, H, D, NB, B, maxpg, S, nchunk;   // nchunk: plan chunks per sequence
  int RD;                     // rotary dims: the first RD of each head (multiple of 16)
  int any_window;             // some layer has a sliding window
};

// Element strides of the K/V pools: page, kv head, layer.  One (layer, page,
// head) chunk is 16*D contiguous values.
#ifndef AKV_HEAD_MAJOR
#define AKV_HEAD_MAJOR 0
#endif
struct PoolStrides {
  size_t page, head, layer;
};
__host__ __device__ inline PoolStrides pool_strides(int NB, int H, int D) {
  const size_t chunk = (size_t)kPage * D;
#if AKV_HEAD_MAJOR
  return PoolStrides{chunk, (size_t)NB * chunk, (size_t)H * NB * chunk};   // [L][H][NB][16][D]
#else
  return PoolStrides{(size_t)H * chunk, chunk, (size_t)NB * H * chunk};    // [L][NB][H][16][D]
#endif
}

// Position of entry j of a sequence whose page-table row is trow.
__device__ __forceinline__ int entry_pos(const Dev &d, const int32_t *trow, int j) {
  return d.pos[(size_t)trow[j >> 4] * kPage + (j & 15)];
}

// First index j in [a, b) whose position is >= lo (b if none).  A sequence's
// positions strictly increase with the index (append counts up, drop keeps
// order, reposition requires increasing targets), so the test is monotone:
// a 64-way search by the calling wave, two dependent loads per round.  Every
// lane of the wave must call it; the result is the same in every lane.
__device__ inline int first_pos_at_least(const Dev &d, const int32_t *trow, int a, int b,
                                         int lo) {
  const int lane = threadIdx.x & 63;
  while (b - a > 64) {
    const int step = (b - a + 63) / 64;            // probes a, a+step, ..., a+63*step >= b-1
    const int j = a + lane * step;
    const bool ge = j >= b || entry_pos(d, trow, j) >= lo;
    const unsigned long long m = __ballot(ge);
    if (m == 0ull) {
      a += 63 * step + 1;                          // every probe is in range and below lo
    } else {
      const int t = __ffsll(m) - 1;                // first probe at or past the answer
      b = min(b, a + t * step);
      if (t) a += (t - 1) * step + 1;
    }
  }
  const int j = a + lane;
  const bool below = j < b && entry_pos(d, trow, j) < lo;
  return a + __popcll(__ballot(below));
}

// Scratch layout (byte offsets from the scratch base, each 256-B aligned).
struct ScratchLayout {
  size_t ctl, theta, seq_info, src_map, delta_map, stage, chunk_info, fork_dst, window, last_src,
      groups, share, ex_list, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

constexpr int kPlanChunkPages = 256;   // pages per plan workgroup

inline int plan_chunks(int maxpg) { return (maxpg + kPlanChunkPages - 1) / kPlanChunkPages; }

inline ScratchLayout scratch_layout(int B, int S, int NB, int L) {
  ScratchLayout s;
  size_t o = 0;
  s.ctl = o;       o = align256(o + CTL_COUNT * 4);
  s.theta = o;     o = align256(o + kMaxHalf * 8);
  s.seq_info = o;  o = align256(o + size_t(B) * kSeqInfo * 4);
  s.src_map = o;   o = align256(o + size_t(B) * S * 4);
  s.delta_map = o; o = align256(o + size_t(B) * S * 4);
  s.stage = o;     o = align256(o + size_t(NB) * 4);
  s.chunk_info = o; o = align256(o + size_t(B) * plan_chunks(S / kPage) * 2 * 4);
  s.fork_dst = o;  o = align256(o + size_t(B) * 4);
  s.window = o;    o = align256(o + size_t(L) * 4);
  s.last_src = o;  o = align256(o + size_t(B) * S * 4);
  s.groups = o;    o = align256(o + size_t(kMaxOpGroups) * kGroupRec * 4);
  s.share = o;     o = align256(o + size_t(NB) * 4);
  s.ex_list = o;   o = align256(o + size_t(NB) * 4);
  s.total = o;
  return s;
}

// Launchers (each in the .hip file that defines its kernels).
hipError_t launch_plan(const Dev &d, const uint8_t *mask, const int32_t *new_pos,
                       const int32_t *old_pos, int mode, int max_groups, hipStream_t st);
// group 0: the one-shot launch (oneshot_cap blocks) and, if grid > 0, the
// persistent one; group >= 1: the persistent launch only
hipError_t launch_move(const Dev &d, int mode, int grid, int oneshot_cap, int group,
                       hipStream_t st);
hipError_t launch_commit(const Dev &d, int group, hipStream_t st);
hipError_t launch_fork_map(const Dev &d, const int32_t *dst_of_host, hipStream_t st);
int move_blocks_per_cu(int D, int RD);
hipError_t launch_append(const Dev &d, const int32_t *counts, int64_t n_new,
                         const uint16_t *k_new, const uint16_t *v_new,
                         const int32_t *tok_new, bool rope, hipStream_t st);
hipError_t launch_release(const Dev &d, const uint8_t *sel, hipStream_t st);
hipError_t launch_query(const Dev &d, int32_t *lens, int32_t *next, int32_t *pos, int32_t *tok,
                        int32_t *last_src, hipStream_t st);
hipError_t launch_reset(const Dev &d, const int32_t *order_dev, hipStream_t st);
// Order of a decode call's layers along the grid when some have a sliding
// window: full-attention layers first (passed in kernel arguments).
constexpr int kMaxOrderedLayers = 512;
struct LayerOrder {
  int n;                          // 0: natural order (sequence-major, layers fastest)
  int16_t idx[kMaxOrderedLayers]; // layer offsets within the call, full-attention first
};
hipError_t launch_attention(const Dev &d, const uint16_t *q, const int32_t *active_len,
                            int l0, int nL, int Hq, uint16_t *out, float *part,
                            int nsplit, const LayerOrder &order, hipStream_t st);
int attn_blocks_per_cu(int D);
hipError_t launch_combine(const float *part, uint16_t *out, int rows, int nsplit,
                          int D, hipStream_t st);
hipError_t launch_segment_attention(const Dev &d, const uint16_t *q, const int32_t *seg_seq,
                                    const int32_t *seg_q_off, int n_seg, int max_q, int l0,
                                    int nL, int Hq, uint16_t *out, hipStream_t st);

}  // namespace akv
