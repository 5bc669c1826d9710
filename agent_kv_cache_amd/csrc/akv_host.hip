// Host side of libakv: argument validation, launch planning, the C ABI of
// include/akv.h and optional per-kernel event timing.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <vector>

#include "akv_internal.h"

using akv::Dev;

namespace akv {
int attn_threads();   // work-items per decode workgroup (akv_attn.hip)
}

// Decode workspace of akv_decode_attention_noalloc, for callers that cannot
// allocate: one fixed array in the library's code object, so every GPU the
// library runs on holds its own copy until the process ends.  In host code
// this name is only a stand-in for the symbol; the device address of each
// GPU's copy comes from hipGetSymbolAddress (static_scratch_ptr below) and is
// the only form ever passed to a kernel.
static __device__ __align__(256) char scratch[AKV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on `device`, looked up once per device with
// that device current (akv_cache_init calls it for the caller's device).
hipError_t static_scratch_ptr(int device, void **out) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device) return hipErrorInvalidDevice;
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = p;
  }
  *out = g_scratch_ptr[device];
  return hipSuccess;
}

}  // namespace

struct akv_cache {
  akv_cache_desc desc;
  Dev dev;
  akv::ScratchLayout layout;
  int device = 0;
  int n_cu = 256;
  int move_grid = 2048;
  int oneshot_cap = 1;     // blocks of the one-shot move launch (the largest op it moves)
  long long layer_groups = 1;   // one-shot blocks per rebuilt page
  bool move_persistent = true;   // some op could be too large for the one-shot launch
  int attn_per_cu = 2;
  int op_groups = 1;       // (move, commit) rounds of a drop / reposition (1: the pool always fits)
  int n_full_layers = 0;   // layers without a sliding window
  void *noalloc_ws = nullptr;   // this device's copy of `scratch`
  std::vector<int32_t> window;  // per-layer sliding window (host copy)
  bool profile = false;
  struct Rec {
    int kernel;
    hipEvent_t a, b;
  };
  std::vector<Rec> pending;
  std::vector<hipEvent_t> spare;
  double total_ms[AKV_KERNEL_COUNT] = {};
  int64_t launches[AKV_KERNEL_COUNT] = {};
};

namespace {

#define AKV_HIP(expr)                           \
  do {                                          \
    if ((expr) != hipSuccess) return AKV_ERR_HIP; \
  } while (0)

hipEvent_t take_event(akv_cache *c) {
  if (!c->spare.empty()) {
    hipEvent_t e = c->spare.back();
    c->spare.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Records an event pair around one launch when profiling is on.
struct Timed {
  akv_cache *c;
  int kernel;
  hipStream_t st;
  hipEvent_t a = nullptr, b = nullptr;
  Timed(akv_cache *c_, int k, hipStream_t s) : c(c_), kernel(k), st(s) {
    if (c->profile) {
      a = take_event(c);
      b = take_event(c);
      if (a && b) {
        (void)hipEventRecord(a, st);
      } else {
        // (one of the two could not be created: time nothing, keep the other)
        if (a) c->spare.push_back(a);
        if (b) c->spare.push_back(b);
        a = b = nullptr;
      }
    }
  }
  ~Timed() {
    if (a && b) {
      (void)hipEventRecord(b, st);
      c->pending.push_back({kernel, a, b});
    }
  }
};

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Split count of the decode grid.  The host never reads device lengths, so
// the choice uses only (sequences x layers x kv heads) rows and the resident
// capacity (workgroups per CU from the occupancy API x CUs): at least one
// full round, and among up to 4x that many splits the one whose last round of
// workgroups is fullest (ties: fewer splits, less combine work).  Each split's
// page range is then cut on the device from the actual length.
int nsplit_for(const akv_cache *c, int nL) {
#ifdef AKV_DECODE_NSPLIT
  // launch-shape knob: a fixed split count (sweeps)
  return std::max(1, std::min(AKV_DECODE_NSPLIT, std::max(1, c->desc.max_blocks_per_seq / 4)));
#endif
  // Rows that carry the work: with sliding-window layers the full-attention
  // layers dominate (a window row reads at most W entries), so the split
  // count is sized for their share of the layers.
  long long lay = nL;
  if (c->n_full_layers < c->desc.n_layers && c->n_full_layers > 0)
    lay = std::max(1LL, ((long long)nL * c->n_full_layers + c->desc.n_layers - 1) /
                            c->desc.n_layers);
  const long long rows = (long long)c->desc.n_seqs * lay * c->desc.n_kv_heads;
  const long long cap = (long long)c->attn_per_cu * c->n_cu;
  const long long max_ns = std::max(1, c->desc.max_blocks_per_seq / 4);
  const long long ns_min = std::min(max_ns, std::max(1LL, (cap + rows - 1) / rows));
  long long best = ns_min;
  double best_eff = 0.0;
  for (long long ns = ns_min; ns <= std::min(max_ns, 4 * ns_min); ++ns) {
    const long long wg = rows * ns;
    const long long rounds = (wg + cap - 1) / cap;
    const double eff = (double)wg / (double)(rounds * cap);
    if (eff > best_eff + 1e-9) {
      best_eff = eff;
      best = ns;
    }
  }
  return (int)best;
}

// One drop / reposition / fork: the plan, then one (move, commit) round per
// sequence group.  A fork copies without freeing anything, so it is never
// split; other ops get c->op_groups rounds (rounds past the groups the plan
// made exit at once).
akv_status run_compaction(akv_cache *c, const uint8_t *mask, const int32_t *new_pos,
                          const int32_t *old_pos, int mode, void *stream,
                          long long max_pages = -1) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int rounds = (mode & akv::M_FORK) ? 1 : c->op_groups;
  // a one-sequence cache is committed by the plan (one group, no fork)
  if (c->desc.n_seqs == 1) mode |= akv::M_STAGED;
  {
    Timed tm(c, AKV_KERNEL_PLAN, st);
    AKV_HIP(akv::launch_plan(c->dev, mask, new_pos, old_pos, mode, rounds, st));
  }
  // the persistent grid is needed only if this call could rebuild more
  // (page, layer group) units than the one-shot grid holds: the cache-wide
  // bound, or the caller's per-call bound (a fork copies at most
  // max_blocks_per_seq pages per source), which also trims the one-shot grid
  // (its blocks past the op's units only exit)
  bool persistent = c->move_persistent;
  int cap = c->oneshot_cap;
  if (max_pages >= 0) {
    persistent = max_pages * c->layer_groups > c->oneshot_cap;
    if (!persistent) cap = (int)std::max(1LL, max_pages * c->layer_groups);
  }
  {
    Timed tm(c, AKV_KERNEL_MOVE, st);
    AKV_HIP(akv::launch_move(c->dev, mode, persistent ? c->move_grid : 0, cap, 0, st));
  }
  if (!(mode & akv::M_STAGED)) {
    Timed tm(c, AKV_KERNEL_COMMIT, st);
    AKV_HIP(akv::launch_commit(c->dev, 0, st));
  }
  if (rounds > 1) {
    Timed tm(c, AKV_KERNEL_ROUNDS, st);
    for (int g = 1; g < rounds; ++g) {
      AKV_HIP(akv::launch_move(c->dev, mode, c->move_grid, c->oneshot_cap, g, st));
      AKV_HIP(akv::launch_commit(c->dev, g, st));
    }
  }
  return AKV_OK;
}

}  // namespace

extern "C" {

size_t akv_scratch_bytes(const akv_cache_desc *d) {
  if (!d || d->n_seqs < 1 || d->max_blocks_per_seq < 1 || d->n_blocks < 1) return 0;
  if (d->n_layers < 1) return 0;
  return akv::scratch_layout(d->n_seqs, d->max_blocks_per_seq * akv::kPage, d->n_blocks,
                             d->n_layers).total;
}

akv_status akv_cache_init(const akv_cache_desc *d, akv_cache **out) {
  if (!d || !out) return AKV_ERR_ARG;
  *out = nullptr;
  if (d->n_layers < 1 || d->n_kv_heads < 1 || d->n_blocks < 1 || d->n_seqs < 1 ||
      d->max_blocks_per_seq < 1)
    return AKV_ERR_ARG;
  // the plan and state-export grids index sequences on their second axis
  if (d->n_seqs > 65535) return AKV_ERR_ARG;
  if (d->block_size != akv::kPage) return AKV_ERR_ARG;
  if (d->head_dim != 64 && d->head_dim != 128) return AKV_ERR_ARG;
  // rotation frequencies must lie in [0, 1] (rope_base >= 1): the move's sine
  // and cosine reduce angles delta * theta_i below 2^31 exactly
  if (!(d->rope_base >= 1.0) || !isfinite(d->rope_base)) return AKV_ERR_ARG;
  if ((long long)d->max_blocks_per_seq * akv::kPage > INT32_MAX / 2) return AKV_ERR_ARG;
  if (!d->k_pool || !d->v_pool || !d->block_table || !d->seq_lens || !d->next_pos ||
      !d->positions || !d->token_ids || !d->free_stack || !d->free_count || !d->scratch)
    return AKV_ERR_ARG;
  if (!aligned(d->k_pool, 16) || !aligned(d->v_pool, 16) || !aligned(d->scratch, 256) ||
      !aligned(d->positions, 16) || !aligned(d->token_ids, 16))
    return AKV_ERR_ARG;
  if (d->scratch_bytes < akv_scratch_bytes(d)) return AKV_ERR_ARG;
  const int rd = d->rotary_dim ? d->rotary_dim : d->head_dim;
  if (rd < 16 || rd > d->head_dim || rd % 16) return AKV_ERR_ARG;
  if (d->inv_freq)
    for (int i = 0; i < rd / 2; ++i)
      if (!isfinite(d->inv_freq[i]) || d->inv_freq[i] < 0.0 || d->inv_freq[i] > 1.0)
        return AKV_ERR_ARG;
  int any_window = 0;
  if (d->layer_window)
    for (int l = 0; l < d->n_layers; ++l) {
      if (d->layer_window[l] < 0) return AKV_ERR_ARG;
      any_window |= d->layer_window[l] > 0;
    }

  akv_cache *c = new (std::nothrow) akv_cache();
  if (!c) return AKV_ERR_ARG;
  c->desc = *d;
  const int S = d->max_blocks_per_seq * akv::kPage;
  c->layout = akv::scratch_layout(d->n_seqs, S, d->n_blocks, d->n_layers);
  char *sb = static_cast<char *>(d->scratch);
  Dev &v = c->dev;
  v.k = d->k_pool;
  v.v = d->v_pool;
  v.table = d->block_table;
  v.lens = d->seq_lens;
  v.next_pos = d->next_pos;
  v.pos = d->positions;
  v.tok = d->token_ids;
  v.free_stack = d->free_stack;
  v.free_count = d->free_count;
  v.ctl = reinterpret_cast<int32_t *>(sb + c->layout.ctl);
  v.theta = reinterpret_cast<const double *>(sb + c->layout.theta);
  v.seq_info = reinterpret_cast<int32_t *>(sb + c->layout.seq_info);
  v.src_map = reinterpret_cast<int32_t *>(sb + c->layout.src_map);
  v.delta_map = reinterpret_cast<int32_t *>(sb + c->layout.delta_map);
  v.stage = reinterpret_cast<int32_t *>(sb + c->layout.stage);
  v.chunk_info = reinterpret_cast<int32_t *>(sb + c->layout.chunk_info);
  v.fork_dst = reinterpret_cast<int32_t *>(sb + c->layout.fork_dst);
  v.window = reinterpret_cast<const int32_t *>(sb + c->layout.window);
  v.last_src = reinterpret_cast<int32_t *>(sb + c->layout.last_src);
  v.groups = reinterpret_cast<int32_t *>(sb + c->layout.groups);
  v.share = reinterpret_cast<int32_t *>(sb + c->layout.share);
  v.ex_list = reinterpret_cast<int32_t *>(sb + c->layout.ex_list);
  v.RD = rd;
  v.any_window = any_window;
  c->n_full_layers = d->n_layers;
  if (d->layer_window)
    for (int l = 0; l < d->n_layers; ++l) c->n_full_layers -= d->layer_window[l] > 0;
  v.L = d->n_layers;
  v.H = d->n_kv_heads;
  v.D = d->head_dim;
  v.NB = d->n_blocks;
  v.B = d->n_seqs;
  v.maxpg = d->max_blocks_per_seq;
  v.S = S;
  v.nchunk = akv::plan_chunks(d->max_blocks_per_seq);

  if (hipGetDevice(&c->device) != hipSuccess ||
      hipDeviceGetAttribute(&c->n_cu, hipDeviceAttributeMultiprocessorCount, c->device) !=
          hipSuccess ||
      static_scratch_ptr(c->device, &c->noalloc_ws) != hipSuccess) {
    delete c;
    return AKV_ERR_HIP;
  }
  c->move_grid = akv::move_blocks_per_cu(d->head_dim, rd) * c->n_cu;
  {
    // One-shot launch size: every block the op could need (one per layer
    // group of each page it could rebuild), at most AKV_MOVE_ONESHOT_CAP
    // blocks; blocks past the planned count exit at once and a larger op runs
    // on the persistent grid.
    const long long pages = std::min<long long>(d->n_blocks,
                                                (long long)d->n_seqs * d->max_blocks_per_seq);
    const int lpb = AKV_MOVE_OS_LAYERS > 0 ? AKV_MOVE_OS_LAYERS : (d->head_dim == 128 ? 1 : 2);
    const long long groups = (d->n_layers + lpb - 1) / lpb;
    c->layer_groups = groups;
    long long cap = AKV_MOVE_ONESHOT_CAP;
    if (const char *e = getenv("AKV_MOVE_ONESHOT_CAP")) cap = std::max(0LL, atoll(e));
    c->oneshot_cap = (int)std::max(1LL, std::min<long long>(pages * groups, cap));
    c->move_persistent = pages * groups > c->oneshot_cap;
  }
  c->attn_per_cu = akv::attn_blocks_per_cu(d->head_dim);
  {
    // A drop / reposition needs at most as many fresh pages as the sequences
    // hold; when the table can address more than half the pool, the pool may
    // run short and the op may have to run in sequence groups: up to
    // AKV_MAX_OP_GROUPS rounds (environment, else the compile-time default).
    long long g = AKV_MAX_OP_GROUPS;
    if (const char *e = getenv("AKV_MAX_OP_GROUPS")) g = atoll(e);
    g = std::max(1LL, std::min<long long>({g, (long long)akv::kMaxOpGroups, d->n_seqs}));
    const bool may_run_short = 2LL * d->n_seqs * d->max_blocks_per_seq > d->n_blocks;
    c->op_groups = may_run_short ? (int)g : 1;
  }

  // theta_i over the rotary dims: the caller's table, else base^(-2i/r);
  // double, uploaded once.  Per-layer windows likewise.
  double theta[akv::kMaxHalf] = {};
  for (int i = 0; i < rd / 2; ++i)
    theta[i] = d->inv_freq ? d->inv_freq[i] : pow(d->rope_base, -2.0 * (double)i / (double)rd);
  std::vector<int32_t> win(d->n_layers, 0);
  if (d->layer_window) std::copy(d->layer_window, d->layer_window + d->n_layers, win.begin());
  c->window = win;
  if (hipMemcpy(sb + c->layout.theta, theta, sizeof(theta), hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(sb + c->layout.window, win.data(), sizeof(int32_t) * win.size(),
                hipMemcpyHostToDevice) != hipSuccess) {
    delete c;
    return AKV_ERR_HIP;
  }
  *out = c;
  return AKV_OK;
}

void akv_cache_free(akv_cache *c) {
  if (!c) return;
  for (auto &r : c->pending) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  for (auto e : c->spare) (void)hipEventDestroy(e);
  delete c;
}

akv_status akv_cache_reset(akv_cache *c, const int32_t *page_order, void *stream) {
  if (!c) return AKV_ERR_ARG;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int NB = c->desc.n_blocks;
  const int32_t *order_dev = nullptr;
  if (page_order) {
    std::vector<char> seen(NB, 0);
    for (int i = 0; i < NB; ++i) {
      const int32_t p = page_order[i];
      if (p < 0 || p >= NB || seen[p]) return AKV_ERR_ARG;
      seen[p] = 1;
    }
    AKV_HIP(hipStreamSynchronize(st));
    AKV_HIP(hipMemcpy(c->dev.stage, page_order, sizeof(int32_t) * NB, hipMemcpyHostToDevice));
    order_dev = c->dev.stage;
  }
  AKV_HIP(akv::launch_reset(c->dev, order_dev, st));
  return AKV_OK;
}

static akv_status append_impl(akv_cache *c, const int32_t *counts, int64_t n_new,
                              const uint16_t *k_new, const uint16_t *v_new,
                              const int32_t *token_ids, bool rope, void *stream) {
  if (!c || !counts || n_new < 0 || n_new > INT32_MAX) return AKV_ERR_ARG;
  if (n_new > 0 && (!k_new || !v_new || !token_ids)) return AKV_ERR_ARG;
  if (n_new > 0 && (!aligned(k_new, 16) || !aligned(v_new, 16))) return AKV_ERR_ARG;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  Timed tm(c, AKV_KERNEL_APPEND, st);
  AKV_HIP(akv::launch_append(c->dev, counts, n_new, k_new, v_new, token_ids, rope, st));
  return AKV_OK;
}

akv_status akv_append(akv_cache *c, const int32_t *counts, int64_t n_new, const uint16_t *k_new,
                      const uint16_t *v_new, const int32_t *token_ids, void *stream) {
  return append_impl(c, counts, n_new, k_new, v_new, token_ids, false, stream);
}

akv_status akv_append_rope(akv_cache *c, const int32_t *counts, int64_t n_new,
                           const uint16_t *k_raw, const uint16_t *v_new, const int32_t *token_ids,
                           void *stream) {
  return append_impl(c, counts, n_new, k_raw, v_new, token_ids, true, stream);
}

akv_status akv_release(akv_cache *c, const uint8_t *release, void *stream) {
  if (!c || !release) return AKV_ERR_ARG;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  Timed tm(c, AKV_KERNEL_RELEASE, st);
  AKV_HIP(akv::launch_release(c->dev, release, st));
  return AKV_OK;
}

akv_status akv_query_state(akv_cache *c, int32_t *seq_lens, int32_t *next_pos,
                           int32_t *positions, int32_t *token_ids, int32_t *last_src,
                           void *stream) {
  if (!c) return AKV_ERR_ARG;
  if (!seq_lens && !next_pos && !positions && !token_ids && !last_src) return AKV_OK;
  AKV_HIP(akv::launch_query(c->dev, seq_lens, next_pos, positions, token_ids, last_src,
                            reinterpret_cast<hipStream_t>(stream)));
  return AKV_OK;
}

akv_status akv_drop(akv_cache *c, const uint8_t *drop_mask, void *stream) {
  if (!c || !drop_mask || !aligned(drop_mask, 16)) return AKV_ERR_ARG;
  return run_compaction(c, drop_mask, nullptr, nullptr, akv::M_DROP, stream);
}

akv_status akv_reposition(akv_cache *c, const int32_t *old_pos, const int32_t *new_pos,
                          void *stream) {
  if (!c || (old_pos && !aligned(old_pos, 16)) || (new_pos && !aligned(new_pos, 16)))
    return AKV_ERR_ARG;
  int mode = akv::M_REPOS;
  if (new_pos) mode |= akv::M_NEWPOS;
  if (old_pos) mode |= akv::M_OLDPOS;
  return run_compaction(c, nullptr, new_pos, old_pos, mode, stream);
}

akv_status akv_drop_reposition(akv_cache *c, const uint8_t *drop_mask, const int32_t *new_pos,
                               void *stream) {
  if (!c || !drop_mask || !aligned(drop_mask, 16) || (new_pos && !aligned(new_pos, 16)))
    return AKV_ERR_ARG;
  int mode = akv::M_DROP | akv::M_REPOS;
  if (new_pos) mode |= akv::M_NEWPOS;
  return run_compaction(c, drop_mask, new_pos, nullptr, mode, stream);
}

akv_status akv_fork(akv_cache *c, const int32_t *dst_of, const uint8_t *drop_mask, int reposition,
                    const int32_t *new_pos, void *stream) {
  if (!c || !dst_of) return AKV_ERR_ARG;
  if ((drop_mask && !aligned(drop_mask, 16)) || (new_pos && !aligned(new_pos, 16)))
    return AKV_ERR_ARG;
  if (new_pos && !reposition) return AKV_ERR_ARG;
  const int B = c->desc.n_seqs;
  std::vector<char> is_dst(B, 0), is_src(B, 0);
  int n = 0;
  for (int b = 0; b < B; ++b) {
    const int e = dst_of[b];
    if (e < -1 || e >= B || e == b) return AKV_ERR_ARG;
    if (e >= 0) {
      if (is_dst[e]) return AKV_ERR_ARG;
      is_dst[e] = 1;
      is_src[b] = 1;
      ++n;
    }
  }
  for (int b = 0; b < B; ++b)
    if (is_dst[b] && is_src[b]) return AKV_ERR_ARG;   // a destination may not be forked from
  if (n == 0) return AKV_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  // the map travels in kernel arguments: nothing reads dst_of after return
  AKV_HIP(akv::launch_fork_map(c->dev, dst_of, st));
  int mode = akv::M_FORK;
  if (drop_mask) mode |= akv::M_DROP;
  if (reposition) mode |= akv::M_REPOS;
  if (new_pos) mode |= akv::M_NEWPOS;
  return run_compaction(c, drop_mask, new_pos, nullptr, mode, stream,
                        (long long)n * c->desc.max_blocks_per_seq);
}

size_t akv_decode_workspace_bytes(const akv_cache *c, int32_t n_layers, int32_t n_q_heads) {
  if (!c || n_layers < 1 || n_q_heads < 1) return 0;
  const int ns = nsplit_for(c, n_layers);
  if (ns == 1) return 256;
  return akv::align256((size_t)c->desc.n_seqs * n_layers * n_q_heads * ns *
                       (size_t)(c->desc.head_dim + 2) * sizeof(float));
}

static akv_status decode_impl(akv_cache *c, const uint16_t *q, const int32_t *active_len,
                              int32_t layer_begin, int32_t n_layers, int32_t n_q_heads,
                              uint16_t *out, void *workspace, size_t workspace_bytes,
                              bool static_ws, void *stream) {
  if (!c || !q || !out) return AKV_ERR_ARG;
  if (layer_begin < 0 || n_layers < 1 || layer_begin + n_layers > c->desc.n_layers)
    return AKV_ERR_ARG;
  if (n_q_heads < 1 || n_q_heads % c->desc.n_kv_heads != 0 ||
      n_q_heads / c->desc.n_kv_heads > 16)
    return AKV_ERR_ARG;
  if (!aligned(q, 16) || !aligned(out, 2)) return AKV_ERR_ARG;
  const int ns = nsplit_for(c, n_layers);
  // one-dimensional grids: (split, kv head, sequence, layer) workgroups for
  // the decode, (sequence, layer, query head) ones for the combine; each
  // launch's size in work-items must fit 32 bits
  const long long rows = (long long)c->desc.n_seqs * n_layers;
  if (rows * ns * c->desc.n_kv_heads * akv::attn_threads() > (long long)UINT32_MAX ||
      rows * n_q_heads * c->desc.head_dim > (long long)UINT32_MAX)
    return AKV_ERR_ARG;
  if (ns > 1) {
    const size_t need = akv_decode_workspace_bytes(c, n_layers, n_q_heads);
    if (static_ws) {
      if (need > (size_t)AKV_NOALLOC_SCRATCH_BYTES) return AKV_ERR_SCRATCH;
      if (!c->noalloc_ws) return AKV_ERR_HIP;
      workspace = c->noalloc_ws;
    } else if (!workspace || workspace_bytes < need) {
      return AKV_ERR_ARG;
    }
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  // full-attention layers first along the grid when the call mixes them
  // with sliding-window layers (natural order otherwise)
  akv::LayerOrder order;
  order.n = 0;
  if (n_layers <= akv::kMaxOrderedLayers) {
    int nfull = 0, nwin = 0;
    for (int li = 0; li < n_layers; ++li) (c->window[layer_begin + li] ? nwin : nfull) += 1;
    if (nwin && nfull) {
      int k = 0;
      for (int pass = 0; pass < 2; ++pass)
        for (int li = 0; li < n_layers; ++li)
          if ((c->window[layer_begin + li] != 0) == (pass == 1)) order.idx[k++] = (int16_t)li;
      order.n = n_layers;
    }
  }
  {
    Timed tm(c, AKV_KERNEL_ATTN, st);
    AKV_HIP(akv::launch_attention(c->dev, q, active_len, layer_begin, n_layers, n_q_heads, out,
                                  static_cast<float *>(workspace), ns, order, st));
  }
  if (ns > 1) {
    Timed tm(c, AKV_KERNEL_COMBINE, st);
    AKV_HIP(akv::launch_combine(static_cast<float *>(workspace), out,
                                c->desc.n_seqs * n_layers * n_q_heads, ns, c->desc.head_dim, st));
  }
  return AKV_OK;
}

akv_status akv_decode_attention(akv_cache *c, const uint16_t *q, const int32_t *active_len,
                                int32_t layer_begin, int32_t n_layers, int32_t n_q_heads,
                                uint16_t *out, void *workspace, size_t workspace_bytes,
                                void *stream) {
  return decode_impl(c, q, active_len, layer_begin, n_layers, n_q_heads, out, workspace,
                     workspace_bytes, false, stream);
}

akv_status akv_decode_attention_noalloc(akv_cache *c, const uint16_t *q,
                                        const int32_t *active_len, int32_t layer_begin,
                                        int32_t n_layers, int32_t n_q_heads, uint16_t *out,
                                        void *stream) {
  return decode_impl(c, q, active_len, layer_begin, n_layers, n_q_heads, out, nullptr, 0, true,
                     stream);
}

akv_status akv_segment_attention(akv_cache *c, const uint16_t *q, const int32_t *seg_seq,
                                 const int32_t *seg_q_off, int32_t n_segments, int32_t max_q,
                                 int32_t layer_begin, int32_t n_layers, int32_t n_q_heads,
                                 uint16_t *out, void *stream) {
  if (!c || n_segments < 0) return AKV_ERR_ARG;
  if (n_segments == 0) return AKV_OK;
  if (!q || !out || !seg_seq || !seg_q_off || max_q < 1) return AKV_ERR_ARG;
  if (layer_begin < 0 || n_layers < 1 || layer_begin + n_layers > c->desc.n_layers)
    return AKV_ERR_ARG;
  if (n_q_heads < 1 || n_q_heads % c->desc.n_kv_heads != 0 ||
      n_q_heads / c->desc.n_kv_heads > 16)
    return AKV_ERR_ARG;
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(seg_seq, 4) || !aligned(seg_q_off, 4))
    return AKV_ERR_ARG;
  const int tb = 16 / (n_q_heads / c->desc.n_kv_heads);
  if (n_segments > 65535 || (long long)n_layers * c->desc.n_kv_heads > 65535 ||
      (max_q + (long long)tb - 1) / tb > 0x7fffffff)
    return AKV_ERR_ARG;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  Timed tm(c, AKV_KERNEL_SEGMENT, st);
  AKV_HIP(akv::launch_segment_attention(c->dev, q, seg_seq, seg_q_off, n_segments, max_q,
                                        layer_begin, n_layers, n_q_heads, out, st));
  return AKV_OK;
}

akv_status akv_sync_status(akv_cache *c, void *stream) {
  if (!c) return AKV_ERR_ARG;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  AKV_HIP(hipStreamSynchronize(st));
  int32_t err = 0;
  AKV_HIP(hipMemcpy(&err, c->dev.ctl + akv::CTL_ERR, sizeof(err), hipMemcpyDeviceToHost));
  if (err) {
    const int32_t zero = 0;
    AKV_HIP(hipMemcpy(c->dev.ctl + akv::CTL_ERR, &zero, sizeof(zero), hipMemcpyHostToDevice));
  }
  return static_cast<akv_status>(err);
}

const char *akv_status_string(akv_status s) {
  switch (s) {
    case AKV_OK: return "ok";
    case AKV_ERR_ARG: return "invalid argument";
    case AKV_ERR_ORDER: return "new positions must be >= 0 and strictly increasing";
    case AKV_ERR_POS_MISMATCH: return "old positions differ from the stored positions";
    case AKV_ERR_NO_BLOCKS: return "free page pool too small";
    case AKV_ERR_CAPACITY: return "sequence exceeds max_blocks_per_seq";
    case AKV_ERR_HIP: return "HIP runtime error";
    case AKV_ERR_SCRATCH: return "call needs more than the library's static scratch";
  }
  return "unknown status";
}

akv_status akv_profile_enable(akv_cache *c, int on) {
  if (!c) return AKV_ERR_ARG;
  c->profile = on != 0;
  return AKV_OK;
}

akv_status akv_profile_read(akv_cache *c, int kernel, double *total_ms, int64_t *launches,
                            int reset) {
  if (!c || kernel < 0 || kernel >= AKV_KERNEL_COUNT) return AKV_ERR_ARG;
  // pairs are folded in and recycled one at a time, so a failure leaves only
  // the unread ones pending (none is counted twice)
  size_t done = 0;
  akv_status st = AKV_OK;
  for (; done < c->pending.size(); ++done) {
    const auto &r = c->pending[done];
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
      st = AKV_ERR_HIP;
      break;
    }
    c->total_ms[r.kernel] += ms;
    c->launches[r.kernel] += 1;
    c->spare.push_back(r.a);
    c->spare.push_back(r.b);
  }
  c->pending.erase(c->pending.begin(), c->pending.begin() + done);
  if (st != AKV_OK) return st;
  if (total_ms) *total_ms = c->total_ms[kernel];
  if (launches) *launches = c->launches[kernel];
  if (reset) {
    std::fill(c->total_ms, c->total_ms + AKV_KERNEL_COUNT, 0.0);
    std::fill(c->launches, c->launches + AKV_KERNEL_COUNT, 0);
  }
  return AKV_OK;
}

}  // extern "C"
