// mk_host.cpp - the C ABI: handle, weight repacking, schedule building and
// caching, the decode-step launch, and a host model of the schedule.
//
// Scheduling follows Cohere's North Mini Code megakernel post (Chinese
// version, task-scheduler section): the host builds named waves per layer,
// orders them (qkv -> router -> top-k -> attention -> MoE up/down -> O-proj ->
// RMSNorm), flattens them into one list and places task k on compute unit
// k mod n_cu; attention and MoE work whose size is only known at run time is
// taken by a fixed number of claimer tasks from shared queues. Schedules are
// prebuilt per (batch, context bucket) and picked at each step (engine
// section: select_schedule(max_live_context()) before every launch).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <memory>
#include <random>
#include <string>
#include <vector>

#include "../../include/mk.h"
#include "mk_internal.h"
#include "mk_launch.h"

namespace {

thread_local std::string g_create_error;

// ------------------------------------------------------------------ schedule

struct Schedule {
  int B = 0, bucket = 0;
  int n_splits_full = 0, n_splits_win = 0, pps = 16;
  int pps_full = 16;  // pages per split of full-attention layers (pps unless the fused MoE runs)
  int n_router = 0, n_oproj = 0, n_up_claimers = 0, n_down_claimers = 0, n_lm = 0;
  std::vector<int> n_qkv;  // QKV tasks per kv group
  std::vector<int> n_attn_claimers;  // per layer
  std::vector<int> moe_fixed;        // per layer: MoE claimers with fixed shares
  std::vector<int> moe_fused;        // per layer: fused MoE claimers (their count), 0 otherwise
  int n_ctr = 0;
  // counter layout
  int c_resid0 = 0, c_lm = 0, c_layer0 = 0, c_per_layer = 0;
  // flattened list, its waves (for kernel-per-op) and per-CU lists
  std::vector<mk_task> flat;
  std::vector<int> flat_wave;
  std::vector<mk_task> cu_tasks;
  std::vector<int32_t> cu_off;
  std::vector<std::pair<int, int>> waves;  // [begin, end) into flat
  std::vector<int> flat_unit;              // the unit each flat task runs on
  // device copies
  mk_task* d_cu_tasks = nullptr;
  int32_t* d_cu_off = nullptr;
  mk_task* d_flat = nullptr;
};

// Counters of one layer (indices into the counter array).
struct CtrIdx {
  int qkv;       // [KVH] QKV tasks done per kv group
  int attn;      // [B][KVH] attention splits done per (sequence, group)
  int comb;      // [KVH] combined attention outputs per group
  int router;    // router tasks done
  int route;     // route finalized (1)
  int attn_claim;  // claim counter of the attention split queue
  int up_claim, down_claim;  // claim counters of the two expert queues
  int up_done;   // [E] up/gate items done per active expert slot
  int colblk;    // [NB] contributions per residual column block
  int fin;       // fused MoE: claimers and O projections done (dense: the FFN claimers)
  int mid;       // dense: O projections done (the mid residual's wait)
  int midres;    // dense: mid residual column blocks done (the FFN's input)
  int oproj_claim;  // claiming MoE: claim counter of the O-projection items
};

mk_task make_task(int op, int layer) {
  mk_task t;
  std::memset(&t, 0, sizeof(t));
  t.op = op;
  t.layer = layer;
  for (int i = 0; i < 3; ++i) {
    t.wait_ctr[i] = -1;
    t.wait_tgt[i] = 0;
  }
  t.sig_ctr[0] = t.sig_ctr[1] = -1;
  return t;
}

void add_wait(mk_task& t, int c, int tgt) {
  for (int i = 0; i < 3; ++i)
    if (t.wait_ctr[i] < 0) {
      t.wait_ctr[i] = c;
      t.wait_tgt[i] = tgt;
      return;
    }
  std::abort();
}

}  // namespace

// Offsets (bytes) of the per-step scratch buffers inside one block, the same
// for the handle's allocation and for the static array of the allocation-free
// step; `ctr` (one counter set) and `total` count only in the static array.
struct ScratchLayout {
  size_t h, ssq, u, q, o, part, ao, rp, tki, tkw, route, gu, dn, mp, lmv, lma, qt, kvt, rpt, err, ctr, total;
};

struct mk_handle {
  mk_config cfg{};
  ScratchLayout lay{};
  void* static_scratch = nullptr;  // this device's static scratch array (device address)
  bool static_used = false;        // an allocation-free step ran (its error word is checked too)
  int wave_order = MK_ORDER_SHIPPED;
  int placement = MK_PLACE_TUNED;
  uint64_t place_seed = 1;  // MK_PLACE_RANDOM's seed
  int device = 0;
  bool host_only = false;
  int n_cu = 0;       // compute units
  int n_workers = 0;  // resident workgroups: MK_WGS_PER_CU per compute unit
  std::string err;
  // derived
  int G = 0, qkv_dim = 0, q_dim = 0, kv_dim = 0, e_pad = 0;
  int max_splits = 0, n_lm_tasks = 0, lm_np = 2;
  int CB = 64, NB = 32, router_np = 2, router_ks = 4, n_router_tasks = 0;
  // device memory
  uint16_t* w_all = nullptr;
  size_t s_wqkv = 0, s_wo = 0, s_wr = 0, s_wgu_l = 0, s_wgu_e = 0, s_wd_l = 0, s_wd_e = 0;
  uint16_t *emb = nullptr, *gamma = nullptr, *gamma2 = nullptr, *wqkv = nullptr, *wo = nullptr, *wr = nullptr,
           *wgu = nullptr, *wd = nullptr, *wlm = nullptr;
  // FP8 feed-forward weights (cfg.ffn_fp8): codes in bytes, scales in floats
  uint8_t *wgu8 = nullptr, *wd8 = nullptr, *wd8p = nullptr;
  float* fsc = nullptr;
  size_t s_gu8_l = 0, s_gu8_e = 0, s_d8_l = 0, s_d8_e = 0, s_fsc_l = 0, s_fsc_e = 0;
  float* rope = nullptr;
  uint16_t* kv = nullptr;
  bool kv_owned = false;  // the pool was allocated by mk_create (kv_pool NULL)
  size_t kv_bytes = 0;
  void* scratch = nullptr;
  uint16_t* u = nullptr;
  uint16_t* o = nullptr;
  uint64_t* qt = nullptr;  // tagged queries (batches up to MK_FUSED_B)
  float *h = nullptr, *q = nullptr, *part = nullptr, *ao = nullptr, *ssq = nullptr, *rp = nullptr,
        *tk_w = nullptr, *gu = nullptr, *dn = nullptr, *mp = nullptr, *lm_val = nullptr;
  int32_t *tk_idx = nullptr, *route = nullptr, *lm_arg = nullptr;
  uint32_t* ctr[2] = {nullptr, nullptr};
  int n_ctr_cap = 0;
  uint32_t* err_word = nullptr;
  int32_t* wg_off_identity = nullptr;  // 0..max_tasks for kernel-per-op launches
  int identity_len = 0;
  std::vector<bool> layer_loaded;
  std::vector<bool> ffn_loaded;  // FP8 feed-forward weights of each layer (cfg.ffn_fp8)
  bool globals_loaded = false;
  uint64_t steps = 0;
  uint32_t epoch = 0;  // the last step's epoch in the handle's scratch (tags of tagged hand-offs)
  bool last_tagged = false;  // the last step handed its queries to attention as tagged words
  bool poison = false;       // debug: fill the step's scratch with NaN before each step
  int64_t timeout_ticks = 200000000;  // 2 s at 100 MHz
  int32_t* tk_trace = nullptr;
  uint32_t* task_trace = nullptr;
  size_t task_trace_cap = 0;
  std::map<std::pair<int, int>, std::unique_ptr<Schedule>> scheds;
};

namespace {

mk_status fail(mk_handle* h, mk_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  if (h)
    h->err = buf;
  else
    g_create_error = buf;
  return st;
}

#define HIPCHECK(h, call)                                                                    \
  do {                                                                                       \
    hipError_t e_ = (call);                                                                  \
    if (e_ != hipSuccess) return fail((h), MK_ERR_HIP, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Counters of one layer in the order CtrIdx lists them: QKV per group,
// attention per (sequence, group), combine per group, router, route,
// attention claims, up and down claims, up/gate done per expert slot, column
// blocks, fin, mid, midres.
int counters_per_layer(int KVH, int B, int E, int NB) { return KVH + B * KVH + KVH + 5 + E + NB + 4; }

mk_status validate_config(const mk_config* c) {
  if (!c) return fail(nullptr, MK_ERR_INVALID_ARG, "null config");
  if (c->hidden <= 0 || c->hidden % 256 || c->hidden > 2048)
    return fail(nullptr, MK_ERR_UNSUPPORTED, "hidden must be a multiple of 256 and <= 2048");
  if (c->head_dim != 64 && c->head_dim != 128) return fail(nullptr, MK_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (c->n_kv_heads <= 0 || c->n_q_heads <= 0 || c->n_q_heads % c->n_kv_heads)
    return fail(nullptr, MK_ERR_INVALID_ARG, "n_q_heads must be a positive multiple of n_kv_heads");
  if (c->n_kv_heads > MK_MAX_KVH) return fail(nullptr, MK_ERR_UNSUPPORTED, "n_kv_heads must be <= %d", MK_MAX_KVH);
  const int G = c->n_q_heads / c->n_kv_heads;
  if (G > 16 || G * c->head_dim > 1024)
    return fail(nullptr, MK_ERR_UNSUPPORTED, "group size must be <= 16 and group width <= 1024");
  if (c->dense != 0 && c->dense != 1) return fail(nullptr, MK_ERR_INVALID_ARG, "dense must be 0 or 1");
  if (c->ffn_fp8 != 0 && c->ffn_fp8 != 1) return fail(nullptr, MK_ERR_INVALID_ARG, "ffn_fp8 must be 0 or 1");
  if (c->dense) {
    if (c->n_experts != 1 || c->top_k != 1)
      return fail(nullptr, MK_ERR_INVALID_ARG, "a dense model has n_experts = top_k = 1");
    if (c->expert_ffn <= 0 || c->expert_ffn % 128 || c->expert_ffn > MK_MAX_DENSE_F)
      return fail(nullptr, MK_ERR_UNSUPPORTED, "a dense FFN width must be a multiple of 128, <= %d", MK_MAX_DENSE_F);
    if (c->max_batch > MK_FUSED_B)
      return fail(nullptr, MK_ERR_UNSUPPORTED, "dense models decode at most %d sequences per step", MK_FUSED_B);
  } else {
    if (c->n_experts <= 0 || c->n_experts % 8 || c->n_experts > 128)
      return fail(nullptr, MK_ERR_UNSUPPORTED, "n_experts must be a multiple of 8, <= 128");
    if (c->top_k <= 0 || c->top_k > MK_MAX_TOPK || c->top_k > c->n_experts)
      return fail(nullptr, MK_ERR_UNSUPPORTED, "top_k must be in [1, 8]");
    if (c->expert_ffn <= 0 || c->expert_ffn % 128 || c->expert_ffn > 768)
      return fail(nullptr, MK_ERR_UNSUPPORTED, "expert_ffn must be a multiple of 128, <= 768");
  }
  if (c->vocab <= 0 || c->vocab % 16) return fail(nullptr, MK_ERR_UNSUPPORTED, "vocab must be a multiple of 16");
  if (c->n_layers <= 0) return fail(nullptr, MK_ERR_INVALID_ARG, "n_layers must be positive");
  // (a tagged hand-off names its layer in the low 8 bits of the tag, 0 reserved)
  if (c->n_layers > 254) return fail(nullptr, MK_ERR_UNSUPPORTED, "n_layers must be at most 254");
  if (c->page_size != 16) return fail(nullptr, MK_ERR_UNSUPPORTED, "page_size must be 16");
  if (c->window < 0 || c->full_every < 1) return fail(nullptr, MK_ERR_INVALID_ARG, "bad window pattern");
  if (c->max_batch < 1 || c->max_batch > 32) return fail(nullptr, MK_ERR_UNSUPPORTED, "max_batch must be in [1, 32]");
  if (c->max_seq_len < 1) return fail(nullptr, MK_ERR_INVALID_ARG, "max_seq_len must be positive");
  if (c->max_pages_per_seq < ceil_div(c->max_seq_len, c->page_size))
    return fail(nullptr, MK_ERR_INVALID_ARG, "max_pages_per_seq too small for max_seq_len");
  if (c->n_pages < 1) return fail(nullptr, MK_ERR_INVALID_ARG, "n_pages must be positive");
  // device code addresses one layer of the pool with 32-bit byte offsets
  if ((int64_t)c->n_pages * 2 * c->n_kv_heads * c->page_size * c->head_dim * 2 > INT32_MAX)
    return fail(nullptr, MK_ERR_UNSUPPORTED, "one layer of the KV pool must stay below 2 GB");
  if (c->mode != MK_MODE_MEGAKERNEL && c->mode != MK_MODE_KERNEL_PER_OP)
    return fail(nullptr, MK_ERR_INVALID_ARG, "unknown mode");
  if (!(c->rms_eps > 0.f) || !(c->rope_theta > 0.f)) return fail(nullptr, MK_ERR_INVALID_ARG, "bad eps/theta");
  return MK_OK;
}

void derive(mk_handle* h) {
  const mk_config& c = h->cfg;
  h->G = c.n_q_heads / c.n_kv_heads;
  h->q_dim = c.n_q_heads * c.head_dim;
  h->kv_dim = c.n_kv_heads * c.head_dim;
  h->qkv_dim = h->q_dim + 2 * h->kv_dim;
  h->e_pad = ceil_div(c.n_experts, 16) * 16;  // router columns padded to whole panels
  // attention: at least 16 pages per split, more when a context would need
  // more than 256 splits (the combine keeps one factor per split in LDS);
  // a shorter context may take up to 256 splits of 16 pages or more
  const int pages = ceil_div(c.max_seq_len, c.page_size) + 1;
  h->max_splits = std::min(256, ceil_div(pages, 16));
  h->lm_np = 2;
  // LM head: one task per workgroup (fewer for a small vocabulary)
  h->n_lm_tasks = std::min(h->n_workers > 0 ? h->n_workers : 1, ceil_div(c.vocab / 16, 2));
  // residual column blocks of 64 columns (4 panels) when the width allows
  h->CB = c.hidden >= 1024 ? 64 : 32;
  h->NB = c.hidden / h->CB;
  // counters of one step at the largest batch
  h->n_ctr_cap = (c.n_layers + 2) + c.n_layers * counters_per_layer(c.n_kv_heads, c.max_batch, c.n_experts, h->NB);
  // router: 2-panel tasks over K quarters (K halves for a small hidden size)
  h->router_np = 2;
  h->router_ks = c.hidden >= 1024 ? 4 : 2;
  h->n_router_tasks = c.dense ? 0 : ceil_div(h->e_pad / 16, h->router_np) * h->router_ks;
}

int window_of(const mk_config& c, int l) {
  if (c.window == 0) return 0;
  return (l % c.full_every) == c.full_every - 1 ? 0 : c.window;
}

// Pages per attention split for a batch of B sequences up to `len` long:
// about two tasks per workgroup over a layer's (sequence, group) pairs. (Finer splits above MK_FUSED_B tokens, sized per layer
// kind, and claims of several items at a time were measured slower at batch
// 32 over ragged contexts: the expert phase that follows on every unit then
// loses more than the attention gains.)
int pps_for(const mk_handle* h, int B, int len) {
  const int pages = ceil_div(len, h->cfg.page_size) + 1;
  // (a dense model: at most as many splits as units left free by the QKV
  // tasks, one per unit, so no attention claimer starts behind a QKV task and
  // streams its pages late)
  const int units = h->cfg.dense ? h->n_workers - h->qkv_dim / 32 : 2 * h->n_workers;
  const int target = std::max(1, units / (B * h->cfg.n_kv_heads));
  // that many splits, each of 16 pages or more, at most 256 (the combine
  // keeps one factor per split in LDS); the pages spread evenly over them
  // (a last split of a page or two would take a unit of its own for nothing)
  const int ns = std::max(1, std::min({target, pages / 16, 256}));
  int pps = ceil_div(pages, ns);
  // The combine merges up to `cap` splits per round trip to memory; when the
  // split count just passes a multiple of it, splits up to 1/8 longer save
  // that round trip.
  const int gd4 = h->cfg.n_q_heads / h->cfg.n_kv_heads * h->cfg.head_dim / 4;
  const int cap = std::max(1, MK_WG_THREADS / gd4) * MK_COMB_SB;
  const int rounds = ceil_div(ceil_div(pages, pps), cap);
  if (rounds > 1) {
    const int p1 = ceil_div(pages, (rounds - 1) * cap);
    if (8 * p1 <= 9 * pps) pps = p1;
  }
  return pps;
}

// Number of attention splits for a layer when sequences are at most `len` long.
int splits_for(const mk_handle* h, int l, int len, int pps) {
  const int win = window_of(h->cfg, l);
  const int keys = win ? std::min(win, len) : len;
  const int pages = ceil_div(keys, h->cfg.page_size) + 1;  // a window may straddle one extra page
  const int ns = ceil_div(pages, pps);
  // (pps_for keeps a split count within the combine's and the scratch's
  // bound for any length up to the maximum)
  if (ns > h->max_splits) std::abort();
  return ns;
}

int bucket_of(int hint) { return ceil_div(hint, 256) * 256; }

// ------------------------------------------------------------ placements
// Two of the schedulers the megakernel post tried before settling on
// round-robin with tuned wave orders (Chinese version, section on the other
// schedulers it tried): a greedy scheduler that estimates each task's cost
// from the memory it reads, and a brute-force search over random candidates.
// Both re-place the tasks of a schedule built with the tuned rules (the
// claimers' shares are computed there); neither changes what a task does, and
// every list stays in flat order, so any placement decodes the same step and
// cannot deadlock as long as the claimers of one wave sit on distinct units.

static bool is_claimer(int op) { return op == MK_OP_ATTN || op == MK_OP_MOE_FUSED || op == MK_OP_MOE_UP; }

// A candidate of the brute-force search: every wave's tasks over a seeded
// random permutation of the units (task j of a wave on unit perm[j mod n], so
// a wave's claimers stay on distinct units).
void random_placement(const Schedule& S, std::vector<int>& flat_cu, int n_w, uint64_t seed) {
  std::vector<int> perm(n_w);
  for (size_t w = 0; w < S.waves.size(); ++w) {
    std::mt19937_64 rng(seed * 0x9e3779b97f4a7c15ull + w);
    for (int i = 0; i < n_w; ++i) perm[i] = i;
    std::shuffle(perm.begin(), perm.end(), rng);
    for (int k = S.waves[w].first; k < S.waves[w].second; ++k) flat_cu[k] = perm[(k - S.waves[w].first) % n_w];
  }
}

// Bytes a task streams (weights, or keys and values), for the cost model.
static double task_bytes(const mk_handle* h, const Schedule& S, const mk_task& t, int n_claimers) {
  const mk_config& c = h->cfg;
  const double H = c.hidden, panel_row = 16.0 * 2.0;  // a 16-column panel, bytes per row of K
  switch (t.op) {
    case MK_OP_QKV: return t.a[1] * panel_row * H;
    case MK_OP_ROUTER: return t.a[1] * panel_row * (t.a[3] - t.a[2]) * 32.0;
    case MK_OP_OPROJ: return (t.b[1] == 1 ? t.a[3] : 1) * h->CB * 2.0 * h->G * c.head_dim;
    case MK_OP_LMHEAD: return (t.a[1] - t.a[0]) * panel_row * H;
    case MK_OP_ATTN: {
      const double items = (double)S.B * c.n_kv_heads * t.a[3];
      return items / std::max(1, n_claimers) * t.a[4] * c.page_size * c.head_dim * 4.0;
    }
    case MK_OP_MOE_FUSED:
    case MK_OP_MOE_UP: {
      const double e_act = c.dense ? 1.0 : c.n_experts * (1.0 - std::pow(1.0 - (double)c.top_k / c.n_experts, S.B));
      return e_act * 3.0 * H * c.expert_ffn * 2.0 / std::max(1, n_claimers);
    }
    default: return 0.0;
  }
}

// The greedy scheduler: tasks in flat order, each static task on the unit
// where it would finish first under a simple model -- a unit streams 25 GB/s
// while every unit streams, a static task's weights stream before its
// dependency wait, a dependency costs a hop of 4 us (a counter poll and a
// data round trip) after its producers end, and a task's own work 1 us.
// Claimers keep their units (their work is claimed at run time); their
// expected share sets when their unit is free again.
void cost_model_placement(const mk_handle* h, const Schedule& S, std::vector<int>& flat_cu, int n_w) {
  constexpr double kBytesPerUs = 25.0e3, kHopUs = 4.0, kWorkUs = 1.0;
  std::vector<double> cu_free(n_w, 0.0);
  std::vector<std::vector<double>> arr(S.n_ctr);
  // the time a counter reaches `tgt` arrivals (the tgt-th earliest), or its
  // latest arrival when the model counted fewer
  auto reach = [&](int ctr, int tgt) -> double {
    std::vector<double>& v = arr[ctr];
    if (v.empty() || tgt <= 0) return 0.0;
    std::sort(v.begin(), v.end());
    return v[std::min((size_t)tgt, v.size()) - 1];
  };
  // claimers per wave (their shares)
  std::vector<int> wave_n(S.waves.size());
  for (size_t w = 0; w < S.waves.size(); ++w) wave_n[w] = S.waves[w].second - S.waves[w].first;
  const int KVH = h->cfg.n_kv_heads;
  for (size_t k = 0; k < S.flat.size(); ++k) {
    const mk_task& t = S.flat[k];
    double ready = 0.0;
    for (int i = 0; i < 3; ++i)
      if (t.wait_ctr[i] >= 0) ready = std::max(ready, reach(t.wait_ctr[i], t.wait_tgt[i]));
    const double load = task_bytes(h, S, t, wave_n[S.flat_wave[k]]) / kBytesPerUs;
    const double dep = ready > 0.0 ? ready + kHopUs : 0.0;
    int cu = flat_cu[k] >= 0 ? flat_cu[k] : (int)(k % n_w);
    double end;
    if (is_claimer(t.op)) {
      end = std::max(cu_free[cu], dep) + load + kWorkUs;
    } else {
      double best = 1e300;
      for (int c2 = 0; c2 < n_w; ++c2) {
        const double e = std::max(cu_free[c2] + load, dep) + kWorkUs;
        if (e < best - 1e-9) {
          best = e;
          cu = c2;
        }
      }
      end = best;
    }
    flat_cu[k] = cu;
    cu_free[cu] = end;
    // arrivals: the task's signals and the counters its op counts on
    for (int i = 0; i < 2; ++i)
      if (t.sig_ctr[i] >= 0) arr[t.sig_ctr[i]].push_back(end);
    switch (t.op) {
      case MK_OP_OPROJ:
        if (t.b[0] == 1) arr[t.a[2]].push_back(end);
        break;
      case MK_OP_ROUTER: arr[t.a[5]].push_back(end); break;
      case MK_OP_LMHEAD: arr[t.a[3]].push_back(end); break;
      case MK_OP_ATTN: {
        // its share of the (sequence, group, split) items, spread over the groups
        const int items = S.B * KVH * t.a[3], per = (items + wave_n[S.flat_wave[k]] - 1) / wave_n[S.flat_wave[k]];
        for (int g = 0; g < KVH; ++g)
          for (int j = 0; j < (per + KVH - 1) / KVH; ++j) arr[(t.b[0] == 1 ? t.a[5] : t.sig_ctr[0]) + g].push_back(end);
        break;
      }
      default: break;
    }
  }
}

std::unique_ptr<Schedule> build_schedule(const mk_handle* h, int B, int hint) {
  const mk_config& c = h->cfg;
  auto S = std::make_unique<Schedule>();
  S->B = B;
  S->bucket = std::min(bucket_of(hint), c.max_seq_len);
  S->pps_full = pps_for(h, B, S->bucket);
  S->pps = S->pps_full;
  if (B <= MK_FUSED_B && h->n_workers <= MK_WG_THREADS && c.window > 0) {
    // Window layers are split for the window's keys, not the whole context.
    S->pps = pps_for(h, B, std::min(S->bucket, c.window));
    // Fused MoE with a window pattern: full-attention layers get as many
    // splits as the window layers (longer ones), so the same number of
    // compute units holds attention work and the rest share the experts
    // (fewer attention claimers leave more units, and each fewer expert
    // slices, on the chain that sets the layer's time) -- while a split stays
    // within about 512 KiB of keys and values; a longer context is spread
    // over the units as at any batch.
    int lw = 0;
    while (lw < c.n_layers && !window_of(c, lw)) ++lw;
    if (lw < c.n_layers) {
      const int ns_win = splits_for(h, lw, S->bucket, S->pps);
      const int pages = ceil_div(S->bucket, c.page_size) + 1;
      const int page_bytes = c.page_size * c.head_dim * 4;
      const int match_cap = std::max(16, (512 << 10) / page_bytes);
      S->pps_full = std::max(S->pps_full, std::min(ceil_div(pages, std::max(ns_win, 1)), match_cap));
    }
  }
  const int L = c.n_layers, KVH = c.n_kv_heads, E = c.n_experts;
  const int n_w = h->n_workers, NB = h->NB;
  const int kc = c.hidden / 32;

  // counter layout: resid_done[l] for l = 0..L (input of layer l complete;
  // L: the LM head's input), lm, then per layer
  int idx = 0;
  S->c_resid0 = idx;
  idx += L + 1;
  S->c_lm = idx++;
  S->c_layer0 = idx;
  S->c_per_layer = counters_per_layer(KVH, B, E, NB);
  idx += L * S->c_per_layer;
  S->n_ctr = idx;
  auto resid = [&](int l) { return S->c_resid0 + l; };  // input of layer l ready
  auto ci = [&](int l) {
    CtrIdx x;
    int b0 = S->c_layer0 + l * S->c_per_layer;
    x.qkv = b0;
    b0 += KVH;
    x.attn = b0;
    b0 += B * KVH;
    x.comb = b0;
    b0 += KVH;
    x.router = b0++;
    x.route = b0++;
    x.attn_claim = b0++;
    x.up_claim = b0++;
    x.down_claim = b0++;
    x.up_done = b0;
    b0 += E;
    x.colblk = b0;
    b0 += NB;
    x.fin = b0++;
    x.mid = b0++;
    x.midres = b0++;
    x.oproj_claim = b0;
    return x;
  };

  auto begin_wave = [&]() { S->waves.push_back({(int)S->flat.size(), (int)S->flat.size()}); };
  // placement: workgroup `cu`, or (cu < 0) round-robin by flat index
  std::vector<int> flat_cu;
  auto push_at = [&](const mk_task& t, int cu) {
    S->flat.push_back(t);
    S->flat_wave.push_back((int)S->waves.size() - 1);
    S->waves.back().second = (int)S->flat.size();
    flat_cu.push_back(cu);
  };
  auto push = [&](const mk_task& t) { push_at(t, -1); };

  S->n_up_claimers = n_w;
  S->n_down_claimers = n_w;
  const int qkv_np = 2;
  S->n_qkv.assign(KVH, 0);

  // layer 0's input: embedding rows per column block
  begin_wave();
  for (int cb = 0; cb < NB; ++cb) {
    mk_task t = make_task(MK_OP_EMBED, 0);
    t.a[0] = cb;
    t.sig_ctr[0] = resid(0);
    push(t);
  }

  // Fused MoE (at most MK_FUSED_B tokens): the attention splits only count
  // per group and the O projection tasks merge them.
  const bool fused_all = B <= MK_FUSED_B && n_w <= MK_WG_THREADS;
  (void)fused_all;
  // (a dense model's tuned placement is round-robin: the schedule search
  // measured its other rules 6% slower on the dense workload)
  const bool tuned = h->placement != MK_PLACE_ROUND_ROBIN && !(c.dense && h->placement == MK_PLACE_TUNED);
  const bool affinity = h->placement == MK_PLACE_AFFINITY;
  for (int l = 0; l < L; ++l) {
    const CtrIdx x = ci(l);
    auto wait_input = [&](mk_task& t) { add_wait(t, resid(l), NB); };
    // where this layer's tasks went (for the placement of later waves)
    std::vector<int> qkv_cus, attn_cus;
    int n_attn = 0, n_attn_items = 0, attn_flat0 = 0, ns = 0, pps_l = 0;
    int n_free = 0, wa = 256, nt = 0;
    std::vector<char> attn_cu(n_w, 0);
    const bool fused = B <= MK_FUSED_B && n_w <= MK_WG_THREADS;
    // (FP8 feed-forward weights: the claiming MoE at every batch above MK_FUSED_B)
    const bool fixed = B <= 16 && !c.ffn_fp8;
    // the unit a task goes to: `cu` when the placement is tuned, else the
    // round-robin unit of its flat index
    auto place = [&](const mk_task& t, int cu) {
      push_at(t, tuned ? cu : -1);
      return tuned && cu >= 0 ? cu : ((int)S->flat.size() - 1) % n_w;
    };
    // router over K splits; the last one does top-k and route finalize
    auto wave_router = [&]() {
      begin_wave();
      const int rpanels = h->e_pad / 16;
      for (int ks = 0; ks < h->router_ks; ++ks)
        for (int p = 0; p < rpanels; p += h->router_np) {
          mk_task t = make_task(MK_OP_ROUTER, l);
          t.a[0] = p;
          t.a[1] = std::min(h->router_np, rpanels - p);
          t.a[2] = ks * kc / h->router_ks;
          t.a[3] = (ks + 1) * kc / h->router_ks;
          t.a[4] = ks;
          t.a[5] = x.router;
          wait_input(t);
          t.sig_ctr[0] = x.route;
          // (it reads the whole layer input: no single producer to follow)
          place(t, -1);
        }
      S->n_router = h->n_router_tasks;
    };
    // qkv, per kv group: its q heads, its k head, its v head
    auto wave_qkv = [&]() {
      begin_wave();
      for (int g = 0; g < KVH; ++g) {
        const int ranges[3][2] = {{g * h->G * c.head_dim / 16, (g + 1) * h->G * c.head_dim / 16},
                                  {(h->q_dim + g * c.head_dim) / 16, (h->q_dim + (g + 1) * c.head_dim) / 16},
                                  {(h->q_dim + h->kv_dim + g * c.head_dim) / 16,
                                   (h->q_dim + h->kv_dim + (g + 1) * c.head_dim) / 16}};
        int n = 0;
        for (auto& rg : ranges)
          for (int p = rg[0]; p < rg[1]; p += qkv_np) {
            mk_task t = make_task(MK_OP_QKV, l);
            t.a[0] = p;
            t.a[1] = std::min(qkv_np, rg[1] - p);
            t.a[2] = g;
            wait_input(t);
            t.sig_ctr[0] = x.qkv + g;
            qkv_cus.push_back(place(t, -1));
            ++n;
          }
        S->n_qkv[g] = n;
      }
      if (S->n_qkv[KVH - 1] != S->n_qkv[0]) std::abort();
    };
    // attention splits; the last split of a (sequence, group) combines
    auto wave_attn = [&]() {
      begin_wave();
      pps_l = window_of(c, l) ? S->pps : S->pps_full;
      ns = splits_for(h, l, S->bucket, pps_l);
      if (window_of(c, l))
        S->n_splits_win = ns;
      else
        S->n_splits_full = ns;
      // claimers over the (sequence, group, split) queue
      n_attn_items = B * KVH * ns;
      attn_flat0 = (int)S->flat.size();
      S->n_attn_claimers.push_back(std::min(n_w, n_attn_items));
      n_attn = S->n_attn_claimers.back();
      for (int i = 0; i < n_attn; ++i) {
        mk_task t = make_task(MK_OP_ATTN, l);
        t.a[0] = x.attn_claim;
        t.a[1] = x.qkv;
        t.a[2] = S->n_qkv[0];
        t.a[3] = ns;
        t.a[4] = pps_l;
        t.a[5] = x.attn;
        t.b[0] = fused ? 1 : 0;
        t.sig_ctr[0] = x.comb;
        // affinity: on the unit of a QKV task it depends on (claimers of one
        // layer never wait for each other, so two may share a unit)
        const int cu = place(t, affinity && i < (int)qkv_cus.size() ? qkv_cus[i] : -1);
        attn_cus.push_back(cu);
        attn_cu[cu] = 1;
      }
    };
    // the MoE claimers' shares (fixed-share and fused paths)
    auto moe_shares = [&](int moe_flat0) {
      // Fixed shares (at most 16 tokens): the up/gate items go to the
      // claimers whose compute unit (round-robin placement: flat index modulo
      // the workgroups) runs no attention claimer in this layer, when there
      // are enough of them: the split that completes a (sequence, group)
      // merges the splits afterwards, and an up/gate share behind that would
      // hold up the expert's down items. Otherwise every claimer takes a
      // share weighted so that each compute unit streams about the same bytes
      // in this phase: the equal share less the key/value bytes of its
      // attention work (weight wa of 256). Down items are shared equally among
      // the claimers with up/gate work.
      n_free = 0;
      for (int i = 0; i < S->n_up_claimers; ++i) n_free += !attn_cu[(moe_flat0 + i) % n_w];
      const double e_act = E * (1.0 - std::pow(1.0 - (double)c.top_k / E, B));
      const double up_bytes = e_act * 2.0 * c.expert_ffn * c.hidden * 2.0;
      const double kv_per =
          n_attn > 0 ? (double)n_attn_items * pps_l * c.page_size * c.head_dim * 4.0 / n_attn : 0.0;
      const double f = (up_bytes + (S->n_up_claimers - n_free) * kv_per) / S->n_up_claimers;
      wa = f > 0 ? (int)std::lround(256.0 * std::max(0.0, f - kv_per) / f) : 256;
      if (n_free >= n_w / 4) wa = 0;
      if (n_free == 0 && wa == 0) wa = 256;
    };
    // Fused MoE (at most MK_FUSED_B tokens): the same shares over (expert,
    // hidden slice) items; claimers whose share is empty by weight (wa = 0)
    // are left out, and a residual task per column block sums the claimers'
    // rows once all of them and the O projections have arrived.
    auto wave_moe_fused = [&]() {
      begin_wave();
      const int moe_flat0 = (int)S->flat.size();
      moe_shares(moe_flat0);
      nt = wa == 0 ? n_free : S->n_up_claimers;
      S->moe_fused.push_back(nt);
      S->moe_fixed.push_back(0);
      int k_free = 0, k_attn = n_free;
      for (int i = 0; i < S->n_up_claimers; ++i) {
        const int cu = (moe_flat0 + i) % n_w;
        if (wa == 0 && attn_cu[cu]) continue;
        mk_task t = make_task(MK_OP_MOE_FUSED, l);
        t.b[0] = attn_cu[cu] ? k_attn++ : k_free++;
        t.b[1] = n_free;
        t.b[2] = nt;
        t.b[3] = wa;
        add_wait(t, resid(l), NB);
        add_wait(t, x.router, h->n_router_tasks);
        t.sig_ctr[0] = x.fin;
        place(t, cu);
      }
      if (k_free + k_attn - n_free != nt) std::abort();
    };
    // O projection per (group, two column blocks) when that gives at most one
    // task per attention unit's worth of pairs, so each unit's weights stream
    // before its wait; on the units that ran the layer's attention
    std::vector<int> oproj_cus;
    auto wave_oproj_fused = [&]() {
      begin_wave();
      int n_oproj = 0;
      const int per = (NB % 2 == 0 && KVH * NB / 2 <= n_attn) ? 2 : 1;
      for (int g = 0; g < KVH; ++g)
        for (int cb = 0; cb < NB; cb += per) {
          mk_task t = make_task(MK_OP_OPROJ, l);
          t.a[0] = g;
          t.a[1] = cb;
          t.a[2] = c.dense ? x.mid : x.fin;
          t.a[3] = per;
          t.a[4] = ns;
          t.b[0] = 1;
          t.b[1] = 1;  // merges the group's splits itself
          add_wait(t, x.attn + g, B * ns);
          const int cu = place(t, attn_cus[n_oproj % n_attn]);
          if (g == 0)
            for (int k = 0; k < per; ++k) oproj_cus.push_back(cu);
          ++n_oproj;
        }
      S->n_oproj = n_oproj;
    };
    // residual tasks on the units that get no router or QKV task of the next
    // layer (round-robin from the flat index after these tasks), so those
    // tasks' weights still stream before the layer input is ready; with
    // affinity, on the unit of the block's first O projection
    auto wave_residual = [&]() {
      begin_wave();
      int n_qkv_tasks = 0;
      for (int g = 0; g < KVH; ++g) n_qkv_tasks += S->n_qkv[g];
      const int next0 = (int)S->flat.size() + NB + h->n_router_tasks + n_qkv_tasks;
      for (int cb = 0; cb < NB; ++cb) {
        mk_task t = make_task(MK_OP_RESIDUAL, l);
        t.a[0] = cb;
        t.a[1] = c.dense ? MK_RES_DENSE_FFN : MK_RES_PARALLEL;
        t.b[1] = n_free;
        t.b[2] = nt;
        t.b[3] = wa;
        if (c.dense) {
          add_wait(t, x.fin, nt);
        } else {
          add_wait(t, x.fin, nt + S->n_oproj);
          add_wait(t, x.route, 1);
        }
        t.sig_ctr[0] = resid(l + 1);
        place(t, affinity ? oproj_cus[cb] : (next0 + cb) % n_w);
      }
    };
    // Dense layers: the residual after attention (h + the O projections'
    // partials, then the FFN's input with the FFN's gain), one task per
    // column block on the units that ran the O projections
    auto wave_residual_mid = [&]() {
      begin_wave();
      for (int cb = 0; cb < NB; ++cb) {
        mk_task t = make_task(MK_OP_RESIDUAL, l);
        t.a[0] = cb;
        t.a[1] = MK_RES_DENSE_MID;
        t.b[1] = 0;
        t.b[2] = 0;
        t.b[3] = 256;
        add_wait(t, x.mid, S->n_oproj);
        t.sig_ctr[0] = x.midres;
        place(t, oproj_cus[cb % (int)oproj_cus.size()]);
      }
    };
    // Dense layers: the FFN (gate/up, SiLU-and-multiply and down of 16-row
    // slices of its hidden layer: the post's FFN_UPGATE_ACT and FFN_DOWN
    // fused per slice, as the fused MoE does for an expert) in equal
    // contiguous shares over every unit, since attention has finished
    auto wave_ffn_dense = [&]() {
      begin_wave();
      n_free = n_w;
      nt = n_w;
      wa = 256;
      S->moe_fused.push_back(nt);
      S->moe_fixed.push_back(0);
      for (int i = 0; i < n_w; ++i) {
        mk_task t = make_task(MK_OP_MOE_FUSED, l);
        t.b[0] = i;
        t.b[1] = n_free;
        t.b[2] = nt;
        t.b[3] = wa;
        add_wait(t, x.midres, NB);
        t.sig_ctr[0] = x.fin;
        place(t, i);
      }
    };
    // MoE claimers above MK_FUSED_B tokens (fixed shares up to 16, claiming beyond)
    auto wave_moe = [&]() {
      begin_wave();
      const int moe_flat0 = (int)S->flat.size();
      moe_shares(moe_flat0);
      S->moe_fused.push_back(0);
      S->moe_fixed.push_back(fixed ? 1 : 0);
      int k_free = 0, k_attn = n_free;
      for (int i = 0; i < S->n_up_claimers; ++i) {
        mk_task t = make_task(MK_OP_MOE_UP, l);
        t.a[0] = x.up_claim;
        t.a[1] = x.up_done;
        // items per claim: the expected queue (distinct experts of B tokens'
        // top-k under uniform routing) over the claimers likely free when it
        // opens (those not running attention)
        const double e_act = E * (1.0 - std::pow(1.0 - (double)c.top_k / E, B));
        const int n_early = std::max(1, S->n_up_claimers - n_attn);
        t.a[2] = std::max(1, (int)std::ceil(e_act * 2 * c.expert_ffn / 16 / n_early));
        // then the down items (their last block contribution does the residual)
        t.a[3] = x.down_claim;
        t.a[4] = x.colblk;
        t.sig_ctr[0] = resid(l + 1);
        t.a[5] = -1;
        if (fixed) {
          t.b[0] = attn_cu[(moe_flat0 + i) % n_w] ? k_attn++ : k_free++;
          t.b[1] = n_free;
          t.b[2] = S->n_up_claimers;
          t.b[3] = wa;
          add_wait(t, resid(l), NB);
          add_wait(t, x.router, h->n_router_tasks);
        } else {
          add_wait(t, x.route, 1);
          // the O projection's (group, column block) items, claimed between
          // the up/gate and down phases once the group's output is combined
          t.a[5] = x.oproj_claim;
          t.b[0] = x.comb;
          t.b[1] = B;
        }
        // (one claimer per unit: fixed-share claimers wait for each other's
        // up/gate items)
        place(t, -1);
      }
    };
    // O projection per (group, column block), on the compute units that ran
    // this layer's attention claimers (their MoE shares are empty or light,
    // so the projection does not queue behind expert work)
    auto wave_oproj = [&]() {
      begin_wave();
      int n_oproj = 0;
      for (int g = 0; g < KVH; ++g)
        for (int cb = 0; cb < NB; ++cb) {
          mk_task t = make_task(MK_OP_OPROJ, l);
          t.a[0] = g;
          t.a[1] = cb;
          t.a[2] = x.colblk;
          add_wait(t, x.comb + g, B);
          add_wait(t, x.route, 1);
          t.sig_ctr[0] = resid(l + 1);
          place(t, n_attn > 0 ? attn_cus[n_oproj % n_attn] : -1);
          ++n_oproj;
        }
      S->n_oproj = n_oproj;
    };
    // the layer's waves in the chosen order (megakernel post, Chinese
    // version, section on the task scheduler: the host builds named waves per
    // layer, picks an order and flattens them); a dense layer's in their one
    // order
    if (c.dense) {
      wave_qkv();
      wave_attn();
      wave_oproj_fused();
      wave_residual_mid();
      wave_ffn_dense();
      wave_residual();
      continue;
    }
    if (h->wave_order == MK_ORDER_QKV_FIRST) {
      wave_qkv();
      wave_router();
    } else {
      wave_router();
      wave_qkv();
    }
    wave_attn();
    if (fused) {
      if (h->wave_order == MK_ORDER_ATTENTION_FIRST) {
        wave_oproj_fused();
        wave_moe_fused();
      } else {
        wave_moe_fused();
        wave_oproj_fused();
      }
      wave_residual();
    } else if (!fixed) {
      // (claiming: the O projection is the MoE claimers' item queue)
      wave_moe();
    } else if (h->wave_order == MK_ORDER_ATTENTION_FIRST) {
      wave_oproj();
      wave_moe();
    } else {
      wave_moe();
      wave_oproj();
    }
  }
  // LM head: contiguous panel ranges (whole pairs); the last task picks the
  // greedy tokens
  begin_wave();
  const int n_panels = c.vocab / 16, n_pairs = ceil_div(n_panels, 2);
  S->n_lm = h->n_lm_tasks;
  for (int i = 0; i < S->n_lm; ++i) {
    const int pa = (int)((int64_t)i * n_pairs / S->n_lm), pb = (int)((int64_t)(i + 1) * n_pairs / S->n_lm);
    mk_task t = make_task(MK_OP_LMHEAD, L);
    t.a[0] = 2 * pa;
    t.a[1] = std::min(2 * pb, n_panels);
    t.a[2] = i;
    t.a[3] = S->c_lm;
    add_wait(t, resid(L), NB);
    push(t);
  }

  if (h->placement == MK_PLACE_RANDOM) random_placement(*S, flat_cu, n_w, h->place_seed);
  if (h->placement == MK_PLACE_COST_MODEL) cost_model_placement(h, *S, flat_cu, n_w);
  // per-workgroup lists in flat order (every wait is on an earlier task of
  // the flat list, so the lists cannot deadlock), placed as chosen above
  std::vector<std::vector<mk_task>> per(n_w);
  S->flat_unit.resize(S->flat.size());
  for (size_t k = 0; k < S->flat.size(); ++k) {
    S->flat_unit[k] = flat_cu[k] >= 0 ? flat_cu[k] : (int)(k % n_w);
    per[S->flat_unit[k]].push_back(S->flat[k]);
  }
  S->cu_off.assign(n_w + 1, 0);
  for (int i = 0; i < n_w; ++i) {
    S->cu_off[i + 1] = S->cu_off[i] + (int)per[i].size();
    S->cu_tasks.insert(S->cu_tasks.end(), per[i].begin(), per[i].end());
  }
  return S;
}

// The fixed shares of MoE claimer k (claimers [0, nf) weigh 256 each, the
// rest wa each): up/gate items [lo, hi) of n_items, down items [dlo, dhi) of
// n_down in equal shares over the claimers with up/gate weight. The device
// computes the same.
void fixed_shares(int k, int nf, int nt, int wa, int n_items, int n_down, int& lo, int& hi, int& dlo, int& dhi) {
  auto pre = [&](int j) -> int64_t { return j <= nf ? (int64_t)j * 256 : (int64_t)nf * 256 + (int64_t)(j - nf) * wa; };
  const int64_t tot = pre(nt);
  lo = (int)(n_items * pre(k) / tot);
  hi = (int)(n_items * pre(k + 1) / tot);
  const int nd = wa == 0 ? nf : nt;  // down items: to the same claimers as the up/gate items
  dlo = k < nd ? (int)((int64_t)n_down * k / nd) : 0;
  dhi = k < nd ? (int)((int64_t)n_down * (k + 1) / nd) : 0;
}

// Host model of the device: per-CU in-order lists, counters, claim queues and
// the last-arrival actions, with CUs advancing in a seeded random order.
struct SimCU {
  bool in_claimer = false;
  int pending_item = -1;  // claimed item waiting for its dependency
  int chunk_end = 0;      // attention: end of the current claim
  int phase = 0;          // MoE claimer: 0 up/gate items, 1 down items, 2 fixed-share down pairs,
                          // 3 O-projection items
  int item_end = 0;       // fixed shares: end of this claimer's down items (pending_item: the next)
  int pos = 0;
};

// ------------------------------------------------------- hazard checker
// Read-before-arrive and overwrite-before-read checking with per-buffer tags
// (the megakernel post's warning, Chinese version, barrier section: a wrong
// arrival count lets a reader run ahead of its producer). Every buffer a task
// reads or writes is a tagged region; in flat-list order (the program order
// of the step) each region keeps the writers of its current version and the
// readers since. A task knows a producer has finished when a counter it
// waited for is incremented by that producer (every dependency wait in these
// schedules targets the counter's full count), or transitively through what
// such a producer, or an earlier task on its own unit, knew. A read must know
// every writer of the version it reads; a write must know every reader and
// writer of the version it replaces. Reads are modelled at the point the
// device code issues them: before the task's waits, after its first wait, or
// after all of them. Claimers of one wave exchange data among themselves
// through their own item counters (the up/gate and down phases of the
// claiming MoE, the attention splits a combine merges); those accesses are
// not modelled here (the simulator checks those counts).
namespace {
struct Bits {
  std::vector<uint64_t> w;
  explicit Bits(size_t n = 0) : w((n + 63) / 64, 0ull) {}
  void set(size_t i) { w[i >> 6] |= 1ull << (i & 63); }
  bool has(size_t i) const { return (w[i >> 6] >> (i & 63)) & 1ull; }
  void merge(const Bits& o) {
    for (size_t i = 0; i < w.size(); ++i) w[i] |= o.w[i];
  }
};
// regions: buffer kind x index
enum RegionKind { R_H, R_U, R_SSQ, R_Q, R_KV, R_RP, R_ROUTE, R_PART, R_O, R_AO, R_MP, R_LM, R_KINDS };
const char* kRegionName[R_KINDS] = {"h", "u", "ssq", "q", "kv", "router partials", "route", "attention partials",
                                    "attention output", "o-proj partials", "claimer rows", "lm candidates"};
struct Access {
  int kind, index;
  bool write;
  int point;     // 0 before the waits, 1 after the first wait, 2 after all
  int ver = -1;  // writes with one version key form one version (default: the task's wave)
};
}  // namespace

mk_status check_hazards(const mk_handle* h, const Schedule& S, uint32_t flags, std::string& rep) {
  const mk_config& c = h->cfg;
  const int n = (int)S.flat.size(), n_w = h->n_workers, NB = h->NB, KVH = c.n_kv_heads, B = S.B;
  const int qpanels = h->q_dim / 16;
  // the tasks that may increment each counter
  std::vector<std::vector<int>> prod(S.n_ctr);
  auto add_prod = [&](int ctr, int k) {
    if (ctr >= 0 && ctr < S.n_ctr) prod[ctr].push_back(k);
  };
  for (int k = 0; k < n; ++k) {
    const mk_task& t = S.flat[k];
    for (int i = 0; i < 2; ++i) add_prod(t.sig_ctr[i], k);
    switch (t.op) {
      case MK_OP_OPROJ:
        if (t.b[1] == 1) add_prod(t.a[2], k);
        break;
      case MK_OP_ROUTER: add_prod(t.a[5], k); break;
      case MK_OP_LMHEAD: add_prod(t.a[3], k); break;
      case MK_OP_ATTN:
        for (int g = 0; g < KVH; ++g) {
          add_prod(t.sig_ctr[0] + g, k);
          if (t.b[0] == 1) add_prod(t.a[5] + g, k);
        }
        if (t.b[0] != 1)
          for (int i = 0; i < B * KVH; ++i) add_prod(t.a[5] + i, k);
        break;
      default: break;
    }
  }
  // the previous task on each task's unit
  std::vector<int> prev(n, -1), last(n_w, -1);
  for (int k = 0; k < n; ++k) {
    prev[k] = last[S.flat_unit[k]];
    last[S.flat_unit[k]] = k;
  }
  // what each task knows: after its first wait and after all (K1, K2); a
  // counter's union is formed once its producers all precede the waiter
  std::vector<Bits> K(n, Bits(n)), K1(n, Bits(n));
  std::vector<Bits> cunion(S.n_ctr);
  std::vector<char> cdone(S.n_ctr, 0);
  int skipped = 0;
  auto counter_union = [&](int ctr, int waiter) -> const Bits* {
    for (int p : prod[ctr])
      if (p >= waiter || S.flat_wave[p] == S.flat_wave[waiter]) return nullptr;  // within a wave
    if (!cdone[ctr]) {
      cunion[ctr] = Bits(n);
      for (int p : prod[ctr]) {
        cunion[ctr].set(p);
        cunion[ctr].merge(K[p]);
      }
      cdone[ctr] = 1;
    }
    return &cunion[ctr];
  };
  std::vector<Bits> K0(n, Bits(n));  // before the waits: the unit's earlier tasks and what they knew
  for (int k = 0; k < n; ++k) {
    const mk_task& t = S.flat[k];
    if (prev[k] >= 0) {
      K0[k] = K[prev[k]];
      K0[k].set(prev[k]);
    }
    K1[k] = K0[k];
    K[k] = K0[k];
    bool first = true;
    // the device waits on wait_ctr[1] first where an op does (the residual's
    // route), else in index order; K1 holds what the first wait gives
    const int order_res[3] = {1, 0, 2}, order_std[3] = {0, 1, 2};
    const int* ord = t.op == MK_OP_RESIDUAL ? order_res : order_std;
    for (int j = 0; j < 3; ++j) {
      const int i = ord[j];
      if (t.wait_ctr[i] < 0) continue;
      // (a planted schedule mistake, to test the checker: the residual tasks'
      // wait for their contributions left out)
      if ((flags & MK_CHECK_PLANT_MISSING_WAIT) && t.op == MK_OP_RESIDUAL && i == 0) continue;
      const Bits* u = counter_union(t.wait_ctr[i], k);
      if (!u) {
        ++skipped;
        continue;
      }
      K[k].merge(*u);
      if (first) K1[k].merge(*u);
      first = false;
    }
    // an attention claimer waits, per item, for the QKV tasks of the item's
    // group (a[1] + g, count a[2]); it may take an item of any group
    if (t.op == MK_OP_ATTN)
      for (int g = 0; g < KVH; ++g) {
        const Bits* u = counter_union(t.a[1] + g, k);
        if (u) K[k].merge(*u);
      }
    // a claiming MoE claimer's O-projection items wait for their group's
    // combined output (b[0] + g, count b[1])
    if (t.op == MK_OP_MOE_UP && t.a[5] >= 0)
      for (int g = 0; g < KVH; ++g) {
        const Bits* u = counter_union(t.b[0] + g, k);
        if (u) K[k].merge(*u);
      }
  }
  // the regions each task touches
  auto accesses = [&](int k) {
    const mk_task& t = S.flat[k];
    std::vector<Access> a;
    const int l = t.layer, par = l & 1, npar = (l + 1) & 1;
    auto all_input = [&](int p, int point) {
      for (int cb = 0; cb < NB; ++cb) {
        a.push_back({R_U, p * NB + cb, false, point});
        a.push_back({R_SSQ, p * NB + cb, false, point});
      }
    };
    auto write_input = [&](int p, int cb) {
      a.push_back({R_H, cb, true, 2});
      a.push_back({R_U, p * NB + cb, true, 2});
      a.push_back({R_SSQ, p * NB + cb, true, 2});
    };
    // above 4 tokens the last contributor to a column block (an O projection
    // or an expert down item, counted on the block's counter) adds the block's
    // residual: one version per layer, whichever task writes it
    auto block_residual = [&](int cb) {
      const int ver = -(l + 2);
      a.push_back({R_H, cb, false, 2, ver});
      a.push_back({R_H, cb, true, 2, ver});
      a.push_back({R_U, npar * NB + cb, true, 2, ver});
      a.push_back({R_SSQ, npar * NB + cb, true, 2, ver});
    };
    switch (t.op) {
      case MK_OP_EMBED: write_input(0, t.a[0]); break;
      case MK_OP_QKV:
        all_input(par, 2);
        a.push_back({t.a[0] < qpanels ? R_Q : R_KV, t.a[0] < qpanels ? t.a[2] : l * KVH + t.a[2], true, 2});
        break;
      case MK_OP_ROUTER:
        all_input(par, 2);
        a.push_back({R_RP, l, true, 2});
        a.push_back({R_ROUTE, l, true, 2});  // the last one's top-k and route
        break;
      case MK_OP_ATTN:
        for (int g = 0; g < KVH; ++g) {
          a.push_back({R_Q, g, false, 2});
          a.push_back({R_KV, l * KVH + g, false, 2});
          a.push_back({R_PART, g, true, 2});
          if (t.b[0] != 1) a.push_back({R_O, g, true, 2});  // the split that completes a group combines
        }
        break;
      case MK_OP_OPROJ: {
        const int g = t.a[0], per = t.b[1] == 1 ? t.a[3] : 1;
        a.push_back({t.b[1] == 1 ? R_PART : R_O, g, false, 2});
        for (int j = 0; j < per; ++j) a.push_back({R_AO, g * NB + t.a[1] + j, true, 2});
        if (t.b[1] != 1) block_residual(t.a[1]);
        break;
      }
      case MK_OP_MOE_FUSED:
        all_input(par, 2);
        if (!c.dense) {
          a.push_back({R_RP, l, false, 2});
        }
        a.push_back({R_MP, t.b[0], true, 2});
        break;
      case MK_OP_MOE_UP:
        all_input(par, 2);
        a.push_back({R_RP, l, false, 2});
        if (t.a[5] >= 0)  // O-projection items
          for (int g = 0; g < KVH; ++g) {
            a.push_back({R_O, g, false, 2});
            for (int cb = 0; cb < NB; ++cb) a.push_back({R_AO, g * NB + cb, true, 2});
          }
        for (int cb = 0; cb < NB; ++cb) block_residual(cb);
        break;
      case MK_OP_RESIDUAL: {
        const int cb = t.a[0], mode = t.a[1];
        const int hpoint = mode == MK_RES_PARALLEL ? ((flags & MK_CHECK_EARLY_STREAM_READ) ? 0 : 1) : 2;
        a.push_back({R_H, cb, false, hpoint});
        if (mode == MK_RES_PARALLEL) a.push_back({R_ROUTE, l, false, 1});
        if (mode != MK_RES_DENSE_FFN)
          for (int g = 0; g < KVH; ++g) a.push_back({R_AO, g * NB + cb, false, 2});
        if (mode != MK_RES_DENSE_MID)
          for (int i = 0; i < t.b[2]; ++i) a.push_back({R_MP, i, false, 2});
        write_input(mode == MK_RES_DENSE_MID ? par : npar, cb);
        break;
      }
      case MK_OP_LMHEAD:
        all_input(c.n_layers & 1, 2);
        a.push_back({R_LM, 0, true, 2});
        break;
      default: break;
    }
    return a;
  };
  // tags in flat order
  struct Tag {
    std::vector<int> writers, readers;
    int ver = -1 << 30;
  };
  std::vector<std::vector<Tag>> tags(R_KINDS);
  const int sizes[R_KINDS] = {NB, 2 * NB, 2 * NB, KVH, c.n_layers * KVH, c.n_layers, c.n_layers, KVH, KVH,
                              KVH * NB, n_w, 1};
  for (int r = 0; r < R_KINDS; ++r) tags[r].resize(sizes[r]);
  int n_bad = 0;
  auto note = [&](const char* what, int k, int other, int kind, int index) {
    if (n_bad++ < 4) {
      const mk_task& t = S.flat[k];
      const mk_task& o = S.flat[other];
      char buf[320];
      std::snprintf(buf, sizeof buf,
                    "%s: task %d (op %d, layer %d, unit %d) and task %d (op %d, layer %d, unit %d) on %s[%d]; ", what,
                    k, t.op, t.layer, S.flat_unit[k], other, o.op, o.layer, S.flat_unit[other], kRegionName[kind],
                    index);
      rep += buf;
    }
  };
  auto knows = [&](int k, int point, int other) {
    if (other == k) return true;
    const Bits& kb = point == 0 ? K0[k] : point == 1 ? K1[k] : K[k];
    return kb.has(other);
  };
  for (int k = 0; k < n; ++k) {
    const int wave = S.flat_wave[k];
    const bool claimer = is_claimer(S.flat[k].op);
    for (const Access& x : accesses(k)) {
      Tag& tg = tags[x.kind][x.index];
      const int ver = x.ver != -1 ? x.ver : wave;
      const bool same_ver = tg.ver == ver;
      if (!x.write) {
        // (within a version: the claimers of a wave, or the contributors to a
        // block, synchronise on their own counters)
        if (!(same_ver && (claimer || x.ver != -1)))
          for (int w : tg.writers)
            if (!knows(k, x.point, w)) note("read before its writer is known to have finished", k, w, x.kind, x.index);
        tg.readers.push_back(k);
      } else {
        if (!same_ver) {
          for (int r : tg.readers)
            if (!knows(k, x.point, r)) note("overwrite before a reader is known to have finished", k, r, x.kind, x.index);
          for (int w : tg.writers)
            if (!knows(k, x.point, w)) note("overwrite before the previous writer is known to have finished", k, w,
                                            x.kind, x.index);
          tg.writers.clear();
          tg.readers.clear();
          tg.ver = ver;
        }
        tg.writers.push_back(k);
      }
    }
  }
  char buf[160];
  std::snprintf(buf, sizeof buf, "%d hazards over %d tasks (%d waits within a wave not modelled)", n_bad, n, skipped);
  rep = n_bad ? rep + buf : std::string("ok: ") + buf;
  return n_bad ? MK_ERR_STATE : MK_OK;
}

mk_status simulate(mk_handle* h, const Schedule& S, const int32_t* n_active, uint64_t seed, int corrupt,
                   std::string& rep) {
  const mk_config& c = h->cfg;
  const int n_cu = h->n_workers, L = c.n_layers, E = c.n_experts, KVH = c.n_kv_heads, NB = h->NB;
  const int F = c.expert_ffn;
  const int up_per_e = 2 * F / 16, down_per_e = NB;
  const int B = S.B;
  std::vector<mk_task> tasks = S.cu_tasks;
  // every counter's final value: the arrivals it must receive
  std::vector<int64_t> want(S.n_ctr, 0);
  for (int l = 0; l <= L; ++l) want[S.c_resid0 + l] = NB;
  want[S.c_lm] = S.n_lm;
  for (int l = 0; l < L; ++l) {
    const int ns = window_of(c, l) ? S.n_splits_win : S.n_splits_full;
    int k = S.c_layer0 + l * S.c_per_layer;
    const bool merged = S.moe_fused[l] > 0;  // the O projection tasks merge the splits
    for (int g = 0; g < KVH; ++g) want[k++] = S.n_qkv[g];
    for (int i = 0; i < B * KVH; ++i) want[k++] = merged ? (i < KVH ? (int64_t)B * ns : 0) : ns;
    for (int g = 0; g < KVH; ++g) want[k++] = merged ? 0 : B;
    want[k++] = h->n_router_tasks;                                  // router tasks
    want[k++] = c.dense ? 0 : 1;                                    // route finalized
    want[k++] = (int64_t)B * KVH * ns + S.n_attn_claimers[l];        // attention claims
    const bool fused = S.moe_fused[l] > 0, claiming = !S.moe_fixed[l] && !fused;
    want[k++] = claiming ? (int64_t)n_active[l] * up_per_e + S.n_up_claimers : 0;
    want[k++] = claiming ? (int64_t)n_active[l] * down_per_e + S.n_up_claimers : 0;
    for (int a = 0; a < E; ++a) want[k++] = (!fused && a < n_active[l]) ? up_per_e : 0;
    for (int cb = 0; cb < NB; ++cb) want[k++] = fused ? 0 : KVH + n_active[l];
    want[k++] = fused ? S.moe_fused[l] + (c.dense ? 0 : S.n_oproj) : 0;  // fused MoE: claimers, O projections
    want[k++] = c.dense ? S.n_oproj : 0;                                  // dense: O projections
    want[k++] = c.dense ? NB : 0;                                         // dense: mid residual blocks
    want[k++] = claiming ? (int64_t)KVH * NB + S.n_up_claimers : 0;         // O-projection item claims
  }
  // a lost signal: the first wait of the first task at or after `corrupt`
  // waits for one arrival more than its counter ever receives
  for (int k = std::max(corrupt, 0); corrupt >= 0 && k < (int)tasks.size(); ++k)
    if (tasks[k].wait_ctr[0] >= 0) {
      tasks[k].wait_tgt[0] = (int32_t)(want[tasks[k].wait_ctr[0]] + 1);
      break;
    }
  std::vector<int64_t> ctr(S.n_ctr, 0);
  std::vector<SimCU> cu(n_cu);
  std::mt19937_64 rng(seed);
  auto waits_met = [&](const mk_task& t) {
    for (int i = 0; i < 3; ++i)
      if (t.wait_ctr[i] >= 0 && ctr[t.wait_ctr[i]] < t.wait_tgt[i]) return false;
    return true;
  };
  // one contribution to a residual column block; the last one signals
  auto block = [&](const mk_task& t, int base, int cb, int l) {
    if (++ctr[base + cb] == KVH + n_active[l]) ctr[t.sig_ctr[0]]++;
  };
  int64_t remaining = (int64_t)tasks.size();
  std::vector<int> order(n_cu);
  for (int i = 0; i < n_cu; ++i) order[i] = i;
  while (remaining > 0) {
    bool progress = false;
    std::shuffle(order.begin(), order.end(), rng);
    for (int k : order) {
      SimCU& u = cu[k];
      const int beg = S.cu_off[k], end = S.cu_off[k + 1];
      if (beg + u.pos >= end) continue;
      const mk_task& t = tasks[beg + u.pos];
      auto done = [&]() {
        u.pos++;
        remaining--;
        progress = true;
      };
      if (!u.in_claimer) {
        if (!waits_met(t)) continue;
        switch (t.op) {
          case MK_OP_EMBED:
          case MK_OP_QKV:
          case MK_OP_MOE_FUSED:
          case MK_OP_RESIDUAL:
            ctr[t.sig_ctr[0]]++;
            done();
            break;
          case MK_OP_ROUTER:
            if (++ctr[t.a[5]] == h->n_router_tasks) ctr[t.sig_ctr[0]]++;
            done();
            break;
          case MK_OP_OPROJ:
            if (t.b[0] == 1)
              ctr[t.a[2]]++;
            else
              block(t, t.a[2], t.a[1], t.layer);
            done();
            break;
          case MK_OP_LMHEAD:
            ctr[t.a[3]]++;
            done();
            break;
          case MK_OP_ATTN:
          case MK_OP_MOE_UP:
            u.in_claimer = true;
            u.phase = 0;
            progress = true;
            break;
          default:
            done();
        }
        continue;
      }
      // claimer step
      const int l = t.layer;
      const int na = n_active[l];
      if (t.op == MK_OP_MOE_UP && S.moe_fixed[l] && u.phase == 0) {
        // fixed shares: the up/gate items at once, then the down items
        const int n_items = na * up_per_e, n_down = na * down_per_e;
        int lo, hi, dlo, dhi;
        fixed_shares(t.b[0], t.b[1], t.b[2], t.b[3], n_items, n_down, lo, hi, dlo, dhi);
        for (int id = lo; id < hi; ++id) ctr[t.a[1] + id / up_per_e]++;
        u.phase = 2;
        u.pending_item = dlo;
        u.item_end = dhi;
        progress = true;
        continue;
      }
      if (t.op == MK_OP_MOE_UP && u.phase == 2) {
        if (u.pending_item >= u.item_end) {
          u.in_claimer = false;
          u.pending_item = -1;
          done();
          continue;
        }
        const int a = u.pending_item / down_per_e, cb = u.pending_item % down_per_e;
        if (ctr[t.a[1] + a] >= up_per_e) {
          block(t, t.a[4], cb, l);
          u.pending_item++;
          progress = true;
        }
        continue;
      }
      if (t.op == MK_OP_ATTN) {
        const int ns = t.a[3], n_items = B * KVH * ns;
        if (u.pending_item < 0) {
          const int id = (int)ctr[t.a[0]]++;
          progress = true;
          if (id >= n_items) {
            u.in_claimer = false;
            done();
          } else {
            u.pending_item = id;
            u.chunk_end = id + 1;
          }
        } else {
          const int bg = u.pending_item / ns, g = bg % KVH;
          if (ctr[t.a[1] + g] >= t.a[2]) {
            if (t.b[0] == 1)
              ctr[t.a[5] + g]++;
            else if (++ctr[t.a[5] + bg] == ns)
              ctr[t.sig_ctr[0] + g]++;
            if (++u.pending_item >= u.chunk_end) u.pending_item = -1;
            progress = true;
          }
        }
      } else if (u.phase == 0) {  // MoE claimer, up/gate items
        const int id = (int)ctr[t.a[0]]++;
        progress = true;
        if (id >= na * up_per_e) {
          u.phase = t.a[5] >= 0 ? 3 : 1;
          u.pending_item = -1;
        } else {
          ctr[t.a[1] + id / up_per_e]++;
        }
      } else if (u.phase == 3) {  // MoE claimer, O-projection items
        if (u.pending_item < 0) {
          const int id = (int)ctr[t.a[5]]++;
          progress = true;
          if (id >= KVH * NB)
            u.phase = 1;
          else
            u.pending_item = id;
        } else if (ctr[t.b[0] + u.pending_item / NB] >= t.b[1]) {
          block(t, t.a[4], u.pending_item % NB, l);
          u.pending_item = -1;
          progress = true;
        }
      } else if (u.pending_item < 0) {  // MoE claimer, down items
        const int id = (int)ctr[t.a[3]]++;
        progress = true;
        if (id >= na * down_per_e) {
          u.in_claimer = false;
          done();
        } else {
          u.pending_item = id;
        }
      } else {
        const int a = u.pending_item / down_per_e, cb = u.pending_item % down_per_e;
        if (ctr[t.a[1] + a] >= up_per_e) {
          block(t, t.a[4], cb, l);
          u.pending_item = -1;
          progress = true;
        }
      }
    }
    if (!progress) {
      char buf[256];
      snprintf(buf, sizeof(buf), "deadlock: %lld tasks left", (long long)remaining);
      rep = buf;
      return MK_ERR_DEVICE_TIMEOUT;
    }
  }
  for (int i = 0; i < S.n_ctr; ++i)
    if (ctr[i] != want[i]) {
      char buf[256];
      snprintf(buf, sizeof(buf), "counter %d ended at %lld, expected %lld", i, (long long)ctr[i], (long long)want[i]);
      rep = buf;
      return MK_ERR_STATE;
    }
  rep = "ok";
  return MK_OK;
}

mk_status get_schedule(mk_handle* h, int B, int hint, Schedule** out) {
  const int bucket = std::min(bucket_of(hint), h->cfg.max_seq_len);
  auto key = std::make_pair(B, bucket);
  auto it = h->scheds.find(key);
  if (it == h->scheds.end()) {
    auto S = build_schedule(h, B, hint);
    if (S->n_ctr > h->n_ctr_cap)
      return fail(h, MK_ERR_UNSUPPORTED, "schedule needs %d counters, capacity %d", S->n_ctr, h->n_ctr_cap);
    if (!h->host_only) {
      HIPCHECK(h, hipSetDevice(h->device));
      HIPCHECK(h, hipMalloc(&S->d_cu_tasks, S->cu_tasks.size() * sizeof(mk_task)));
      HIPCHECK(h, hipMemcpy(S->d_cu_tasks, S->cu_tasks.data(), S->cu_tasks.size() * sizeof(mk_task),
                            hipMemcpyHostToDevice));
      HIPCHECK(h, hipMalloc(&S->d_cu_off, S->cu_off.size() * sizeof(int32_t)));
      HIPCHECK(h, hipMemcpy(S->d_cu_off, S->cu_off.data(), S->cu_off.size() * sizeof(int32_t), hipMemcpyHostToDevice));
      HIPCHECK(h, hipMalloc(&S->d_flat, S->flat.size() * sizeof(mk_task)));
      HIPCHECK(h, hipMemcpy(S->d_flat, S->flat.data(), S->flat.size() * sizeof(mk_task), hipMemcpyHostToDevice));
      int longest = 0;
      for (auto& w : S->waves) longest = std::max(longest, w.second - w.first);
      if (longest + 1 > h->identity_len) {
        if (h->wg_off_identity) hipFree(h->wg_off_identity);
        std::vector<int32_t> id(longest + 1);
        for (int i = 0; i <= longest; ++i) id[i] = i;
        HIPCHECK(h, hipMalloc(&h->wg_off_identity, id.size() * sizeof(int32_t)));
        HIPCHECK(h, hipMemcpy(h->wg_off_identity, id.data(), id.size() * sizeof(int32_t), hipMemcpyHostToDevice));
        h->identity_len = (int)id.size();
      }
    }
    it = h->scheds.emplace(key, std::move(S)).first;
  }
  *out = it->second.get();
  return MK_OK;
}

void free_schedule(Schedule* S) {
  if (S->d_cu_tasks) hipFree(S->d_cu_tasks);
  if (S->d_cu_off) hipFree(S->d_cu_off);
  if (S->d_flat) hipFree(S->d_flat);
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace

bool mk_handle_dims(const mk_handle* h, int* max_batch, int* mpps, int* n_pages, int* vocab) {
  if (!h || h->host_only) return false;
  *max_batch = h->cfg.max_batch;
  *mpps = h->cfg.max_pages_per_seq;
  *n_pages = h->cfg.n_pages;
  *vocab = h->cfg.vocab;
  return true;
}

// =================================================================== C ABI

extern "C" {

const char* mk_last_error(const mk_handle* h) { return h ? h->err.c_str() : g_create_error.c_str(); }

static mk_status create_common(const mk_config* cfg, mk_handle** out) {
  if (!out) return fail(nullptr, MK_ERR_INVALID_ARG, "null out");
  *out = nullptr;
  mk_status st = validate_config(cfg);
  if (st != MK_OK) return st;
  return MK_OK;
}

mk_status mk_create_host_only(const mk_config* cfg, int n_cus, mk_handle** out) {
  mk_status st = create_common(cfg, out);
  if (st != MK_OK) return st;
  if (n_cus < 1 || n_cus > MK_MAX_CUS) return fail(nullptr, MK_ERR_INVALID_ARG, "n_cus out of range");
  auto* h = new mk_handle();
  h->cfg = *cfg;
  h->host_only = true;
  h->n_cu = n_cus;
  h->n_workers = n_cus * MK_WGS_PER_CU;
  derive(h);
  *out = h;
  return MK_OK;
}

mk_status mk_create(const mk_config* cfg, void* kv_pool, size_t kv_pool_bytes, int device, mk_handle** out) {
  mk_status st = create_common(cfg, out);
  if (st != MK_OK) return st;
  const mk_config& c = *cfg;
  const size_t kv_want = (size_t)c.n_layers * c.n_pages * 2 * c.n_kv_heads * c.page_size * c.head_dim * 2;
  if (kv_pool && kv_pool_bytes != kv_want)
    return fail(nullptr, MK_ERR_INVALID_ARG, "kv_pool must be %zu bytes (got %zu)", kv_want, kv_pool_bytes);
  if (!kv_pool && kv_pool_bytes != 0)
    return fail(nullptr, MK_ERR_INVALID_ARG, "kv_pool_bytes must be 0 when the library allocates the pool");
  if ((uintptr_t)kv_pool % 16) return fail(nullptr, MK_ERR_INVALID_ARG, "kv_pool must be 16-byte aligned");
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev)
    return fail(nullptr, MK_ERR_INVALID_ARG, "no HIP device %d", device);
  auto h = std::unique_ptr<mk_handle, void (*)(mk_handle*)>(new mk_handle(), mk_destroy);
  h->cfg = c;
  h->device = device;
  if (hipSetDevice(device) != hipSuccess) return fail(nullptr, MK_ERR_HIP, "hipSetDevice failed");
  int n_cu = 0;
  if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || n_cu < 1)
    return fail(nullptr, MK_ERR_HIP, "cannot query compute units");
  int occ = 0;
  if (mk_interp_occupancy(c.head_dim, &occ) != hipSuccess || occ < MK_WGS_PER_CU)
    return fail(nullptr, MK_ERR_HIP, "interpreter kernel: %d resident workgroups per CU, need %d", occ,
                MK_WGS_PER_CU);
  h->n_cu = std::min(n_cu, MK_MAX_CUS);
  h->n_workers = h->n_cu * MK_WGS_PER_CU;
  derive(h.get());
  if (const char* e = std::getenv("MK_TIMEOUT_MS")) h->timeout_ticks = (int64_t)std::atoll(e) * 100000;

  const int L = c.n_layers, H = c.hidden, E = c.n_experts, F = c.expert_ffn, V = c.vocab;
  // weights
  h->s_wqkv = (size_t)H * h->qkv_dim;
  h->s_wo = (size_t)h->q_dim * H;
  h->s_wr = c.dense ? 0 : (size_t)H * h->e_pad;
  h->s_wgu_e = (size_t)H * 2 * F;
  h->s_wgu_l = h->s_wgu_e * E;
  h->s_wd_e = (size_t)F * H;
  h->s_wd_l = h->s_wd_e * E;
  size_t off = 0;
  auto take = [&](size_t elems) {
    size_t o = off;
    off += align_up(elems, 256);
    return o;
  };
  const size_t o_emb = take((size_t)V * H), o_gamma = take((size_t)(L + 1) * H), o_wlm = take((size_t)H * V);
  const size_t o_wqkv = take(h->s_wqkv * L), o_wo = take(h->s_wo * L), o_wr = take(h->s_wr * L);
  // (FP8 feed-forward weights replace the bf16 ones: codes, 2 per element,
  // and four float scales, 8 elements, per hidden unit)
  const bool fp8 = c.ffn_fp8 != 0;
  const size_t o_wgu = take(fp8 ? 0 : h->s_wgu_l * L), o_wd = take(fp8 ? 0 : h->s_wd_l * L);
  const size_t o_gamma2 = take(c.dense ? (size_t)L * H : 0);
  h->s_gu8_e = fp8 ? (size_t)H * 2 * F : 0;
  h->s_gu8_l = h->s_gu8_e * E;
  h->s_d8_e = fp8 ? (size_t)F * H : 0;
  h->s_d8_l = h->s_d8_e * E;
  h->s_fsc_e = fp8 ? (size_t)F * 4 : 0;
  h->s_fsc_l = h->s_fsc_e * E;
  const size_t o_gu8 = take(h->s_gu8_l * L / 2), o_d8 = take(h->s_d8_l * L / 2), o_fsc = take(h->s_fsc_l * L * 2);
  // (above MK_FUSED_B sequences the claiming MoE reads the down codes as panels)
  const bool panels8 = fp8 && c.max_batch > MK_FUSED_B;
  const size_t o_d8p = take(panels8 ? h->s_d8_l * L / 2 : 0);
  if (hipMalloc(&h->w_all, off * 2) != hipSuccess)
    return fail(nullptr, MK_ERR_OOM, "cannot allocate %.1f GB of weights", off * 2 / 1e9);
  h->emb = h->w_all + o_emb;
  h->gamma = h->w_all + o_gamma;
  h->wlm = h->w_all + o_wlm;
  h->wqkv = h->w_all + o_wqkv;
  h->wo = h->w_all + o_wo;
  h->wr = h->w_all + o_wr;
  h->wgu = h->w_all + o_wgu;
  h->wd = h->w_all + o_wd;
  h->gamma2 = c.dense ? h->w_all + o_gamma2 : nullptr;
  if (fp8) {
    h->wgu8 = (uint8_t*)(h->w_all + o_gu8);
    h->wd8 = (uint8_t*)(h->w_all + o_d8);
    h->fsc = (float*)(h->w_all + o_fsc);
    h->wd8p = panels8 ? (uint8_t*)(h->w_all + o_d8p) : nullptr;
    h->wgu = h->wd = nullptr;
  }
  h->kv_bytes = kv_want;
  if (kv_pool) {
    h->kv = (uint16_t*)kv_pool;
  } else {
    if (hipMalloc(&h->kv, kv_want) != hipSuccess)
      return fail(nullptr, MK_ERR_OOM, "cannot allocate the %.2f GB KV pool", kv_want / 1e9);
    h->kv_owned = true;
    if (hipMemset(h->kv, 0, kv_want) != hipSuccess) return fail(nullptr, MK_ERR_HIP, "KV pool clear");
  }
  h->layer_loaded.assign(L, false);
  h->ffn_loaded.assign(L, !fp8);

  // RoPE table: angle = pos * theta^(-2i/D) in double, cos/sin rounded to float
  {
    const int D = c.head_dim;
    std::vector<float> tab((size_t)c.max_seq_len * D);
    for (int pos = 0; pos < c.max_seq_len; ++pos)
      for (int i = 0; i < D / 2; ++i) {
        const double f = std::pow((double)c.rope_theta, -2.0 * i / D);
        const double ang = (double)pos * f;
        tab[((size_t)pos * (D / 2) + i) * 2 + 0] = (float)std::cos(ang);
        tab[((size_t)pos * (D / 2) + i) * 2 + 1] = (float)std::sin(ang);
      }
    if (hipMalloc(&h->rope, tab.size() * 4) != hipSuccess) return fail(nullptr, MK_ERR_OOM, "rope table");
    if (hipMemcpy(h->rope, tab.data(), tab.size() * 4, hipMemcpyHostToDevice) != hipSuccess)
      return fail(nullptr, MK_ERR_HIP, "rope upload");
  }

  // scratch
  const int Bm = c.max_batch, K = c.top_k, G = h->G, D = c.head_dim, KVH = c.n_kv_heads;
  size_t so = 0;
  auto stake = [&](size_t bytes) {
    size_t o = so;
    so += align_up(bytes, 256);
    return o;
  };
  ScratchLayout& y = h->lay;
  y.h = stake((size_t)Bm * H * 4);
  y.ssq = stake((size_t)2 * Bm * h->NB * 4);
  y.u = stake((size_t)4 * Bm * H * 2);
  y.q = stake((size_t)Bm * h->q_dim * 4);
  y.o = stake((size_t)Bm * h->q_dim * 4);
  y.part = stake((size_t)Bm * KVH * h->max_splits * (G * D + 2 * G) * 4);
  // routing scratch: one region per layer
  y.ao = stake((size_t)KVH * Bm * H * 4);
  y.rp = stake((size_t)L * h->router_ks * Bm * E * 4);
  y.tki = stake((size_t)L * Bm * K * 4);
  y.tkw = stake((size_t)L * Bm * K * 4);
  y.route = stake((size_t)L * MK_ROUTE_INTS(E, Bm) * 4);
  y.gu = stake((size_t)Bm * K * 4 * F * 4);
  y.dn = stake((size_t)Bm * K * H * 4);
  y.mp = stake((size_t)std::max(h->n_workers, 1) * MK_FUSED_B * H * 4);
  y.lmv = stake((size_t)Bm * h->n_lm_tasks * 4);
  y.lma = stake((size_t)Bm * h->n_lm_tasks * 4);
  // tagged hand-offs (batches up to MK_FUSED_B); zero, which no tag equals
  y.qt = stake((size_t)std::min(Bm, MK_FUSED_B) * h->q_dim * 8);
  y.kvt = stake((size_t)std::min(Bm, MK_FUSED_B) * KVH * 2 * D * 8);
  y.rpt = stake((size_t)std::min(Bm, MK_FUSED_B) * E * 4 * 8);
  y.err = stake(16);
  const size_t scratch_bytes = so;
  // counters: capacity for the largest batch
  y.ctr = stake((size_t)h->n_ctr_cap * 4);
  y.total = so;
  if (hipMalloc(&h->scratch, scratch_bytes) != hipSuccess) return fail(nullptr, MK_ERR_OOM, "scratch");
  hipMemset(h->scratch, 0, scratch_bytes);
  char* sb = (char*)h->scratch;
  h->h = (float*)(sb + y.h);
  h->u = (uint16_t*)(sb + y.u);
  h->ssq = (float*)(sb + y.ssq);
  h->q = (float*)(sb + y.q);
  h->o = (uint16_t*)(sb + y.o);
  h->part = (float*)(sb + y.part);
  h->ao = (float*)(sb + y.ao);
  h->rp = (float*)(sb + y.rp);
  h->tk_idx = (int32_t*)(sb + y.tki);
  h->tk_w = (float*)(sb + y.tkw);
  h->route = (int32_t*)(sb + y.route);
  h->gu = (float*)(sb + y.gu);
  h->dn = (float*)(sb + y.dn);
  h->mp = (float*)(sb + y.mp);
  h->lm_val = (float*)(sb + y.lmv);
  h->lm_arg = (int32_t*)(sb + y.lma);
  h->qt = (uint64_t*)(sb + y.qt);
  h->err_word = (uint32_t*)(sb + y.err);
  for (int i = 0; i < 2; ++i) {
    if (hipMalloc(&h->ctr[i], (size_t)h->n_ctr_cap * 4) != hipSuccess) return fail(nullptr, MK_ERR_OOM, "counters");
    hipMemset(h->ctr[i], 0, (size_t)h->n_ctr_cap * 4);
  }
  // this device's static scratch array (the allocation-free step's), looked up
  // once per device with the device current
  if (mk_static_scratch(device, &h->static_scratch) != hipSuccess)
    return fail(nullptr, MK_ERR_HIP, "cannot look up the static scratch array on device %d", device);
  if (hipDeviceSynchronize() != hipSuccess) return fail(nullptr, MK_ERR_HIP, "create sync");
  *out = h.release();
  return MK_OK;
}

void mk_destroy(mk_handle* h) {
  if (!h) return;
  if (!h->host_only) {
    hipSetDevice(h->device);
    hipDeviceSynchronize();
    for (auto& kv : h->scheds) free_schedule(kv.second.get());
    if (h->wg_off_identity) hipFree(h->wg_off_identity);
    if (h->w_all) hipFree(h->w_all);
    if (h->rope) hipFree(h->rope);
    if (h->scratch) hipFree(h->scratch);
    if (h->kv_owned && h->kv) hipFree(h->kv);
    for (auto* c : h->ctr)
      if (c) hipFree(c);
  }
  delete h;
}

// A layer's attention norm gain, QKV and O projections into the library's copy.
static mk_status load_attention(mk_handle* h, int layer, const void* gamma, const void* wqkv, const void* wo,
                                hipStream_t s) {
  const int H = h->cfg.hidden;
  HIPCHECK(h, hipMemcpyAsync(h->gamma + (size_t)layer * H, gamma, (size_t)H * 2, hipMemcpyDeviceToDevice, s));
  HIPCHECK(h, mk_launch_repack((const uint16_t*)wqkv, h->wqkv + layer * h->s_wqkv, H, h->qkv_dim, h->qkv_dim, 0, 1,
                               1, 0, 0, s));
  HIPCHECK(h, mk_launch_repack((const uint16_t*)wo, h->wo + layer * h->s_wo, h->q_dim, H, H, 0, 1, 1, 0, 0, s));
  return MK_OK;
}

// A layer's expert (or dense FFN: one expert) gate, up and down matrices:
// gate and up panels interleaved (gate panel j -> 2j, up panel j -> 2j+1).
static mk_status load_ffn(mk_handle* h, int layer, const void* wg, const void* wu, const void* wd, hipStream_t s) {
  const int H = h->cfg.hidden, E = h->cfg.n_experts, F = h->cfg.expert_ffn;
  HIPCHECK(h, mk_launch_repack((const uint16_t*)wg, h->wgu + layer * h->s_wgu_l, H, F, F, 0, 2, E, (size_t)H * F,
                               h->s_wgu_e, s));
  HIPCHECK(h, mk_launch_repack((const uint16_t*)wu, h->wgu + layer * h->s_wgu_l, H, F, F, 1, 2, E, (size_t)H * F,
                               h->s_wgu_e, s));
  HIPCHECK(h, mk_launch_repack((const uint16_t*)wd, h->wd + layer * h->s_wd_l, F, H, H, 0, 1, E, (size_t)F * H,
                               h->s_wd_e, s));
  return MK_OK;
}

// bf16 feed-forward weights are given with the layer; FP8 ones (cfg.ffn_fp8)
// through mk_load_ffn_fp8, the layer call then passing NULL for them.
static mk_status check_ffn_args(mk_handle* h, const void* wg, const void* wu, const void* wd) {
  if (h->cfg.ffn_fp8) {
    if (wg || wu || wd)
      return fail(h, MK_ERR_INVALID_ARG, "FP8 feed-forward weights load with mk_load_ffn_fp8 (pass NULL here)");
  } else if (!wg || !wu || !wd) {
    return fail(h, MK_ERR_INVALID_ARG, "null weight pointer");
  }
  return MK_OK;
}

mk_status mk_load_ffn_fp8(mk_handle* h, int layer, const void* wg8, const void* wu8, const void* wd8,
                          const float* sg, const float* su, const float* sd, void* stream) {
  if (!h) return MK_ERR_INVALID_ARG;
  if (h->host_only) return fail(h, MK_ERR_STATE, "host-only handle");
  const mk_config& c = h->cfg;
  if (!c.ffn_fp8) return fail(h, MK_ERR_INVALID_ARG, "not an FP8 model (cfg.ffn_fp8 = 0)");
  if (layer < 0 || layer >= c.n_layers) return fail(h, MK_ERR_INVALID_ARG, "layer %d out of range", layer);
  if (!wg8 || !wu8 || !wd8 || !sg || !su || !sd) return fail(h, MK_ERR_INVALID_ARG, "null weight pointer");
  for (const void* p : {wg8, wu8, wd8, (const void*)sg, (const void*)su, (const void*)sd})
    if ((uintptr_t)p % 16) return fail(h, MK_ERR_INVALID_ARG, "weights must be 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  HIPCHECK(h, hipSetDevice(h->device));
  const int H = c.hidden, E = c.n_experts, F = c.expert_ffn;
  // gate and up panels interleaved (gate panel j -> 2j, up panel j -> 2j + 1)
  uint8_t* gu = h->wgu8 + layer * h->s_gu8_l;
  HIPCHECK(h, mk_launch_repack_fp8_panels((const uint8_t*)wg8, gu, H, F, 0, 2, E, (size_t)H * F, h->s_gu8_e, s));
  HIPCHECK(h, mk_launch_repack_fp8_panels((const uint8_t*)wu8, gu, H, F, 1, 2, E, (size_t)H * F, h->s_gu8_e, s));
  HIPCHECK(h, mk_launch_repack_fp8_d((const uint8_t*)wd8, h->wd8 + layer * h->s_d8_l, F, H, E, s));
  if (h->wd8p)
    HIPCHECK(h, mk_launch_repack_fp8_panels((const uint8_t*)wd8, h->wd8p + layer * h->s_d8_l, F, H, 0, 1, E,
                                            (size_t)F * H, h->s_d8_e, s));
  HIPCHECK(h, mk_launch_pack_scales(sg, su, sd, h->fsc + layer * h->s_fsc_l, E * F, s));
  h->ffn_loaded[layer] = true;
  return MK_OK;
}

mk_status mk_load_layer(mk_handle* h, int layer, const void* gamma, const void* wqkv, const void* wo, const void* wr,
                        const void* wg, const void* wu, const void* wd, void* stream) {
  if (!h) return MK_ERR_INVALID_ARG;
  if (h->host_only) return fail(h, MK_ERR_STATE, "host-only handle");
  const mk_config& c = h->cfg;
  if (layer < 0 || layer >= c.n_layers) return fail(h, MK_ERR_INVALID_ARG, "layer %d out of range", layer);
  if (c.dense) return fail(h, MK_ERR_INVALID_ARG, "a dense model's layers load with mk_load_layer_dense");
  mk_status st = check_ffn_args(h, wg, wu, wd);
  if (st != MK_OK) return st;
  if (!gamma || !wqkv || !wo || !wr) return fail(h, MK_ERR_INVALID_ARG, "null weight pointer");
  for (const void* p : {gamma, wqkv, wo, wr, wg, wu, wd})
    if ((uintptr_t)p % 16) return fail(h, MK_ERR_INVALID_ARG, "weights must be 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  HIPCHECK(h, hipSetDevice(h->device));
  const int H = c.hidden, E = c.n_experts;
  st = load_attention(h, layer, gamma, wqkv, wo, s);
  if (st != MK_OK) return st;
  if (h->e_pad == E) {
    HIPCHECK(h, mk_launch_repack((const uint16_t*)wr, h->wr + layer * h->s_wr, H, E, E, 0, 1, 1, 0, 0, s));
  } else {
    // zero columns pad the router to whole 16-column panels; their logits are never read
    uint16_t* tmp = nullptr;
    HIPCHECK(h, hipMallocAsync((void**)&tmp, (size_t)H * h->e_pad * 2, s));
    HIPCHECK(h, hipMemsetAsync(tmp, 0, (size_t)H * h->e_pad * 2, s));
    HIPCHECK(h, hipMemcpy2DAsync(tmp, (size_t)h->e_pad * 2, wr, (size_t)E * 2, (size_t)E * 2, H,
                                 hipMemcpyDeviceToDevice, s));
    HIPCHECK(h, mk_launch_repack(tmp, h->wr + layer * h->s_wr, H, h->e_pad, h->e_pad, 0, 1, 1, 0, 0, s));
    HIPCHECK(h, hipFreeAsync(tmp, s));
  }
  if (!c.ffn_fp8) {
    st = load_ffn(h, layer, wg, wu, wd, s);
    if (st != MK_OK) return st;
  }
  h->layer_loaded[layer] = true;
  return MK_OK;
}

mk_status mk_load_layer_dense(mk_handle* h, int layer, const void* gamma, const void* wqkv, const void* wo,
                              const void* gamma2, const void* wg, const void* wu, const void* wd, void* stream) {
  if (!h) return MK_ERR_INVALID_ARG;
  if (h->host_only) return fail(h, MK_ERR_STATE, "host-only handle");
  const mk_config& c = h->cfg;
  if (!c.dense) return fail(h, MK_ERR_INVALID_ARG, "not a dense model: load layers with mk_load_layer");
  if (layer < 0 || layer >= c.n_layers) return fail(h, MK_ERR_INVALID_ARG, "layer %d out of range", layer);
  mk_status st = check_ffn_args(h, wg, wu, wd);
  if (st != MK_OK) return st;
  if (!gamma || !wqkv || !wo || !gamma2) return fail(h, MK_ERR_INVALID_ARG, "null weight pointer");
  for (const void* p : {gamma, wqkv, wo, gamma2, wg, wu, wd})
    if ((uintptr_t)p % 16) return fail(h, MK_ERR_INVALID_ARG, "weights must be 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  HIPCHECK(h, hipSetDevice(h->device));
  st = load_attention(h, layer, gamma, wqkv, wo, s);
  if (st != MK_OK) return st;
  HIPCHECK(h, hipMemcpyAsync(h->gamma2 + (size_t)layer * c.hidden, gamma2, (size_t)c.hidden * 2,
                             hipMemcpyDeviceToDevice, s));
  if (!c.ffn_fp8) {
    st = load_ffn(h, layer, wg, wu, wd, s);
    if (st != MK_OK) return st;
  }
  h->layer_loaded[layer] = true;
  return MK_OK;
}

mk_status mk_load_globals(mk_handle* h, const void* emb, const void* gamma_f, const void* wlm, void* stream) {
  if (!h) return MK_ERR_INVALID_ARG;
  if (h->host_only) return fail(h, MK_ERR_STATE, "host-only handle");
  if (!emb || !gamma_f || !wlm) return fail(h, MK_ERR_INVALID_ARG, "null weight pointer");
  for (const void* p : {emb, gamma_f, wlm})
    if ((uintptr_t)p % 16) return fail(h, MK_ERR_INVALID_ARG, "weights must be 16-byte aligned");
  const mk_config& c = h->cfg;
  hipStream_t s = (hipStream_t)stream;
  HIPCHECK(h, hipSetDevice(h->device));
  HIPCHECK(h, hipMemcpyAsync(h->emb, emb, (size_t)c.vocab * c.hidden * 2, hipMemcpyDeviceToDevice, s));
  HIPCHECK(h, hipMemcpyAsync(h->gamma + (size_t)c.n_layers * c.hidden, gamma_f, (size_t)c.hidden * 2,
                             hipMemcpyDeviceToDevice, s));
  HIPCHECK(h, mk_launch_repack((const uint16_t*)wlm, h->wlm, c.hidden, c.vocab, c.vocab, 0, 1, 1, 0, 0, s));
  h->globals_loaded = true;
  return MK_OK;
}

mk_status mk_load_weights(mk_handle* h, const mk_weights* w, void* stream) {
  if (!h || !w) return MK_ERR_INVALID_ARG;
  const bool dense = h->cfg.dense != 0;
  if (!w->gamma || !w->wqkv || !w->wo || !(dense ? w->gamma2 : w->wr) ||
      (!h->cfg.ffn_fp8 && (!w->wg || !w->wu || !w->wd)))
    return fail(h, MK_ERR_INVALID_ARG, "null per-layer pointer array");
  mk_status st = mk_load_globals(h, w->emb, w->gamma_f, w->wlm, stream);
  if (st != MK_OK) return st;
  for (int l = 0; l < h->cfg.n_layers; ++l) {
    // (an FP8 model's feed-forward weights load through mk_load_ffn_fp8)
    const void* wg = w->wg ? w->wg[l] : nullptr;
    const void* wu = w->wu ? w->wu[l] : nullptr;
    const void* wd = w->wd ? w->wd[l] : nullptr;
    st = dense ? mk_load_layer_dense(h, l, w->gamma[l], w->wqkv[l], w->wo[l], w->gamma2[l], wg, wu, wd, stream)
               : mk_load_layer(h, l, w->gamma[l], w->wqkv[l], w->wo[l], w->wr[l], wg, wu, wd, stream);
    if (st != MK_OK) return st;
  }
  return MK_OK;
}

// The per-step scratch pointers of P inside a block laid out as h->lay.
static void scratch_at(const mk_handle* h, char* base, mk_params& P) {
  const ScratchLayout& y = h->lay;
  P.h = (float*)(base + y.h);
  P.u = (uint16_t*)(base + y.u);
  P.ssq = (float*)(base + y.ssq);
  P.q = (float*)(base + y.q);
  P.o = (uint16_t*)(base + y.o);
  P.part = (float*)(base + y.part);
  P.ao = (float*)(base + y.ao);
  P.rp = (float*)(base + y.rp);
  P.tk_idx = (int32_t*)(base + y.tki);
  P.tk_w = (float*)(base + y.tkw);
  P.route = (int32_t*)(base + y.route);
  P.gu = (float*)(base + y.gu);
  P.dn = (float*)(base + y.dn);
  P.mp = (float*)(base + y.mp);
  P.lm_val = (float*)(base + y.lmv);
  P.lm_arg = (int32_t*)(base + y.lma);
  P.qt = (uint64_t*)(base + y.qt);
  P.kvt = (uint64_t*)(base + y.kvt);
  P.rpt = (uint64_t*)(base + y.rpt);
  P.err = (uint32_t*)(base + y.err);
}

static void fill_params(mk_handle* h, Schedule* S, int B, int32_t* tokens, const int32_t* bt, int32_t* seq_lens,
                        float* logits, int32_t* next_tokens, uint32_t flags, mk_params& P) {
  const mk_config& c = h->cfg;
  std::memset(&P, 0, sizeof(P));
  P.H = c.hidden;
  P.QH = c.n_q_heads;
  P.KVH = c.n_kv_heads;
  P.D = c.head_dim;
  P.G = h->G;
  P.E = c.n_experts;
  P.K = c.top_k;
  P.F = c.expert_ffn;
  P.V = c.vocab;
  P.L = c.n_layers;
  P.PS = c.page_size;
  P.window = c.window;
  P.full_every = c.full_every;
  P.eps = c.rms_eps;
  P.attn_scale = (float)(1.0 / std::sqrt((double)c.head_dim));
  P.B = B;
  P.mpps = c.max_pages_per_seq;
  P.n_pages = c.n_pages;
  P.max_seq = std::min(S->bucket, c.max_seq_len);
  P.up_items_per_expert = 2 * c.expert_ffn / 16;
  P.down_items_per_expert = h->NB;
  P.CB = h->CB;
  P.NB = h->NB;
  P.n_router_tasks = h->n_router_tasks;
  P.router_ks = h->router_ks;
  P.max_splits = h->max_splits;
  P.n_lm_tasks = S->n_lm;
  P.e_pad = h->e_pad;
  P.emb = h->emb;
  P.gamma = h->gamma;
  P.gamma2 = h->gamma2;
  P.dense = h->cfg.dense;
  P.wqkv = h->wqkv;
  P.s_wqkv = h->s_wqkv;
  P.wo = h->wo;
  P.s_wo = h->s_wo;
  P.wr = h->wr;
  P.s_wr = h->s_wr;
  P.wgu = h->wgu;
  P.s_wgu_l = h->s_wgu_l;
  P.s_wgu_e = h->s_wgu_e;
  P.wd = h->wd;
  P.s_wd_l = h->s_wd_l;
  P.s_wd_e = h->s_wd_e;
  P.ffn_fp8 = h->cfg.ffn_fp8;
  P.wgu8 = h->wgu8;
  P.s_gu8_l = h->s_gu8_l;
  P.s_gu8_e = h->s_gu8_e;
  P.wd8 = h->wd8;
  P.wd8p = h->wd8p;
  P.s_d8_l = h->s_d8_l;
  P.s_d8_e = h->s_d8_e;
  P.fsc = h->fsc;
  P.s_fsc_l = h->s_fsc_l;
  P.s_fsc_e = h->s_fsc_e;
  P.wlm = h->wlm;
  P.rope = h->rope;
  P.kv = h->kv;
  P.s_kv_l = (size_t)c.n_pages * 2 * c.n_kv_heads * c.page_size * c.head_dim;
  P.tokens = tokens;
  P.bt = bt;
  P.seq_lens = seq_lens;
  P.logits = logits;
  P.next_tokens = next_tokens;
  P.flags = flags;
  scratch_at(h, (char*)h->scratch, P);
  P.tk_trace = h->tk_trace;
  P.trace = h->task_trace;
  P.n_ctr = h->n_ctr_cap;  // clear the whole capacity: schedules differ in size
  P.timeout_ticks = h->timeout_ticks;
}

// Epochs 1 .. 2^24 - 1, in turn (0 is never a tag's epoch: scratch starts zeroed).
static std::atomic<uint32_t> g_static_epoch[MK_MAX_DEVICES];
static uint32_t next_epoch(uint32_t* e) {
  *e = *e >= 0xFFFFFFu ? 1u : *e + 1u;
  return *e;
}
static uint32_t next_epoch(std::atomic<uint32_t>* e) {
  uint32_t cur = e->load(), nxt;
  do {
    nxt = cur >= 0xFFFFFFu ? 1u : cur + 1u;
  } while (!e->compare_exchange_weak(cur, nxt));
  return nxt;
}

static hipError_t poison_scratch(const mk_handle* h, char* base, hipStream_t s);

// One decode step; `noalloc`: the allocation-free variant (static scratch,
// counters zeroed by a fill kernel, only cached schedules).
static mk_status decode_step(mk_handle* h, int batch, int32_t* tokens, const int32_t* block_tables,
                             int32_t* seq_lens, int max_seq_len_hint, float* logits, int32_t* next_tokens,
                             uint32_t flags, void* stream, bool noalloc) {
  if (!h) return MK_ERR_INVALID_ARG;
  if (h->host_only) return fail(h, MK_ERR_STATE, "host-only handle");
  const mk_config& c = h->cfg;
  if (batch < 1 || batch > c.max_batch) return fail(h, MK_ERR_INVALID_ARG, "batch %d not in [1, %d]", batch, c.max_batch);
  if (!tokens || !block_tables || !seq_lens || !logits)
    return fail(h, MK_ERR_INVALID_ARG, "null tokens/block_tables/seq_lens/logits");
  if (max_seq_len_hint < 1 || max_seq_len_hint > c.max_seq_len)
    return fail(h, MK_ERR_INVALID_ARG, "max_seq_len_hint %d not in [1, %d]", max_seq_len_hint, c.max_seq_len);
  if (flags & ~MK_STEP_ADVANCE) return fail(h, MK_ERR_INVALID_ARG, "unknown flags");
  if ((flags & MK_STEP_ADVANCE) && max_seq_len_hint >= c.max_seq_len)
    return fail(h, MK_ERR_INVALID_ARG, "advancing past max_seq_len");
  if (!h->globals_loaded) return fail(h, MK_ERR_STATE, "embedding/LM head not loaded");
  for (int l = 0; l < c.n_layers; ++l) {
    if (!h->layer_loaded[l]) return fail(h, MK_ERR_STATE, "layer %d not loaded", l);
    if (!h->ffn_loaded[l]) return fail(h, MK_ERR_STATE, "layer %d: FP8 feed-forward weights not loaded", l);
  }
  Schedule* S = nullptr;
  if (noalloc) {
    if (h->lay.total > MK_STATIC_SCRATCH_BYTES)
      return fail(h, MK_ERR_UNSUPPORTED,
                  "this model and batch need %zu bytes of step scratch; the static array holds %u",
                  h->lay.total, (unsigned)MK_STATIC_SCRATCH_BYTES);
    if (!h->static_scratch) return fail(h, MK_ERR_STATE, "no static scratch on this device");
    const int bucket = std::min(bucket_of(max_seq_len_hint), c.max_seq_len);
    auto it = h->scheds.find(std::make_pair(batch, bucket));
    if (it == h->scheds.end())
      return fail(h, MK_ERR_STATE,
                  "no schedule for batch %d, context bucket %d yet (building one allocates): run "
                  "mk_decode_step or mk_schedule_info_get once with these sizes first",
                  batch, bucket);
    S = it->second.get();
  } else {
    mk_status st = get_schedule(h, batch, max_seq_len_hint, &S);
    if (st != MK_OK) return st;
  }
  if (h->task_trace && S->cu_tasks.size() > h->task_trace_cap)
    return fail(h, MK_ERR_INVALID_ARG, "task trace holds %zu records, the schedule has %zu tasks", h->task_trace_cap,
                S->cu_tasks.size());
  HIPCHECK(h, hipSetDevice(h->device));
  hipStream_t s = (hipStream_t)stream;
  mk_params P;
  fill_params(h, S, batch, tokens, block_tables, seq_lens, logits, next_tokens, flags, P);
  // the lengths limit on the device is the hint (the schedule's splits cover it)
  P.max_seq = max_seq_len_hint;
  uint32_t* clear_next = nullptr;
  // Tagged hand-offs name the step by an epoch that differs from the last
  // one written into the same scratch: per handle, and for the static array
  // (shared by every handle on the device) per device.
  P.tagged = batch <= MK_FUSED_B ? 1 : 0;
  h->last_tagged = P.tagged != 0;
  P.tag_base = (noalloc ? next_epoch(&g_static_epoch[h->device]) : next_epoch(&h->epoch)) << 8;
  if (noalloc) {
    // the static array keeps the last call's contents: only the counters must
    // start at zero (every other buffer is written before it is read)
    char* base = (char*)h->static_scratch;
    scratch_at(h, base, P);
    P.ctr = (uint32_t*)(base + h->lay.ctr);
    P.ctr_clear = nullptr;
    HIPCHECK(h, mk_launch_zero(P.ctr, h->n_ctr_cap, s));
    h->static_used = true;
  } else {
    const int cur = (int)(h->steps & 1), nxt = cur ^ 1;
    P.ctr = h->ctr[cur];
    P.ctr_clear = clear_next = h->ctr[nxt];
  }
  if (h->poison) HIPCHECK(h, poison_scratch(h, noalloc ? (char*)h->static_scratch : (char*)h->scratch, s));
  if (c.mode == MK_MODE_MEGAKERNEL) {
    P.tasks = S->d_cu_tasks;
    P.task_off = S->d_cu_off;
    P.waits_enabled = 1;
    HIPCHECK(h, mk_launch_interp(P, c.head_dim, h->n_workers, true, s));
  } else {
    P.waits_enabled = 0;
    P.task_off = h->wg_off_identity;
    for (size_t w = 0; w < S->waves.size(); ++w) {
      const int b0 = S->waves[w].first, n = S->waves[w].second - S->waves[w].first;
      if (n == 0) continue;
      P.tasks = S->d_flat + b0;
      P.trace_base = b0;
      P.ctr_clear = (w == 0) ? clear_next : nullptr;
      HIPCHECK(h, mk_launch_interp(P, c.head_dim, n, false, s));
    }
  }
  if (!noalloc) h->steps++;
  return MK_OK;
}

mk_status mk_decode_step(mk_handle* h, int batch, int32_t* tokens, const int32_t* block_tables, int32_t* seq_lens,
                         int max_seq_len_hint, float* logits, int32_t* next_tokens, uint32_t flags, void* stream) {
  return decode_step(h, batch, tokens, block_tables, seq_lens, max_seq_len_hint, logits, next_tokens, flags, stream,
                     false);
}

mk_status mk_decode_step_noalloc(mk_handle* h, int batch, int32_t* tokens, const int32_t* block_tables,
                                 int32_t* seq_lens, int max_seq_len_hint, float* logits, int32_t* next_tokens,
                                 uint32_t flags, void* stream) {
  return decode_step(h, batch, tokens, block_tables, seq_lens, max_seq_len_hint, logits, next_tokens, flags, stream,
                     true);
}

mk_status mk_set_task_trace(mk_handle* h, uint32_t* trace, size_t n_records) {  // records of 8 words
  if (!h) return MK_ERR_INVALID_ARG;
  h->task_trace = trace;
  h->task_trace_cap = trace ? n_records : 0;
  return MK_OK;
}

mk_status mk_set_mode(mk_handle* h, int mode) {
  if (!h) return MK_ERR_INVALID_ARG;
  if (mode != MK_MODE_MEGAKERNEL && mode != MK_MODE_KERNEL_PER_OP) return fail(h, MK_ERR_INVALID_ARG, "unknown mode");
  h->cfg.mode = mode;
  return MK_OK;
}

static mk_status drop_schedules(mk_handle* h) {
  if (!h->host_only) {
    HIPCHECK(h, hipSetDevice(h->device));
    HIPCHECK(h, hipDeviceSynchronize());  // no step may still read the old lists
    for (auto& kv : h->scheds) free_schedule(kv.second.get());
  }
  h->scheds.clear();
  return MK_OK;
}

mk_status mk_set_schedule_options(mk_handle* h, int wave_order, int placement) {
  if (!h) return MK_ERR_INVALID_ARG;
  if (wave_order < MK_ORDER_SHIPPED || wave_order > MK_ORDER_ATTENTION_FIRST)
    return fail(h, MK_ERR_INVALID_ARG, "unknown wave order %d", wave_order);
  if (placement < MK_PLACE_TUNED || placement > MK_PLACE_RANDOM)
    return fail(h, MK_ERR_INVALID_ARG, "unknown placement %d", placement);
  if (wave_order == h->wave_order && placement == h->placement) return MK_OK;
  mk_status st = drop_schedules(h);
  if (st != MK_OK) return st;
  h->wave_order = wave_order;
  h->placement = placement;
  return MK_OK;
}

mk_status mk_set_placement_seed(mk_handle* h, uint64_t seed) {
  if (!h) return MK_ERR_INVALID_ARG;
  if (seed == h->place_seed) return MK_OK;
  mk_status st = drop_schedules(h);
  if (st != MK_OK) return st;
  h->place_seed = seed;
  return MK_OK;
}

mk_status mk_set_debug_poison(mk_handle* h, int on) {
  if (!h) return MK_ERR_INVALID_ARG;
  h->poison = on != 0;
  return MK_OK;
}

// Debug poison of one step's scratch block (laid out as h->lay): values NaN
// (float 0xffffffff, bf16 0xffff), index buffers 0, tagged words NaN with tag
// 0 (which no step uses); the error word and the counters are left alone.
static hipError_t poison_scratch(const mk_handle* h, char* base, hipStream_t s) {
  const ScratchLayout& y = h->lay;
  const uint32_t NaN = 0xffffffffu;
  struct Region { size_t off, end; uint32_t lo, hi; };
  const Region rs[] = {
      {y.h, y.tki, NaN, NaN},      // h, ssq, u, q, o, part, ao, rp
      {y.tki, y.tkw, 0u, 0u},      // top-k ids
      {y.tkw, y.route, NaN, NaN},  // top-k weights
      {y.route, y.gu, 0u, 0u},     // routes
      {y.gu, y.lma, NaN, NaN},     // gu, dn, mp, LM-head candidates
      {y.lma, y.qt, 0u, 0u},       // LM-head candidate ids
      {y.qt, y.err, NaN, 0u},      // tagged words
  };
  for (const Region& r : rs) {
    hipError_t e = mk_launch_fill((uint32_t*)(base + r.off), (int)((r.end - r.off) / 4), r.lo, r.hi, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

mk_status mk_set_wait_limit(mk_handle* h, uint32_t microseconds) {
  if (!h) return MK_ERR_INVALID_ARG;
  h->timeout_ticks = microseconds == 0 ? 200000000 : (int64_t)microseconds * 100;  // 100 MHz ticks
  return MK_OK;
}

mk_status mk_stream_read(const void* buf, size_t bytes, void* stream) {
  if (!buf || bytes == 0 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(buf) & 15) != 0)
    return fail(nullptr, MK_ERR_INVALID_ARG, "stream_read: buffer must be 16-byte aligned, bytes a nonzero multiple of 16");
  if (mk_launch_stream_read(buf, bytes / 16, (hipStream_t)stream) != hipSuccess)
    return fail(nullptr, MK_ERR_HIP, "stream_read launch failed");
  return MK_OK;
}

mk_status mk_litmus_message_passing(int device, int pairs, int rounds, int coherent, uint32_t* stale,
                                    uint32_t* timeouts) {
  if (pairs < 1 || pairs > 512 || rounds < 1 || rounds > 1000000 || coherent < 0 || coherent > 2 || !stale ||
      !timeouts)
    return fail(nullptr, MK_ERR_INVALID_ARG,
                "litmus: pairs in [1, 512], rounds in [1, 1e6], coherent in [0, 2], non-null outputs");
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev)
    return fail(nullptr, MK_ERR_INVALID_ARG, "litmus: bad device %d", device);
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return fail(nullptr, MK_ERR_HIP, "hipGetDevice failed");
  if (hipSetDevice(device) != hipSuccess) return fail(nullptr, MK_ERR_HIP, "hipSetDevice failed");
  const size_t words = (size_t)pairs * 64 + 3 * (size_t)pairs * 2;
  uint32_t* buf = nullptr;
  mk_status st = MK_OK;
  std::vector<uint32_t> res(2 * (size_t)pairs, 0);
  if (hipMalloc(&buf, words * 4) != hipSuccess) {
    st = fail(nullptr, MK_ERR_OOM, "litmus buffers");
  } else {
    uint32_t *msg = buf, *flag = buf + (size_t)pairs * 64, *ack = flag + 2 * pairs, *result = ack + 2 * pairs;
    // every wait gives up after 20 ms (2e6 ticks of the 100 MHz clock)
    if (hipMemset(buf, 0, words * 4) != hipSuccess ||
        mk_launch_litmus(msg, flag, ack, result, pairs, rounds, coherent, 2000000, nullptr) != hipSuccess ||
        hipDeviceSynchronize() != hipSuccess ||
        hipMemcpy(res.data(), result, res.size() * 4, hipMemcpyDeviceToHost) != hipSuccess)
      st = fail(nullptr, MK_ERR_HIP, "litmus launch failed");
    (void)hipFree(buf);
  }
  (void)hipSetDevice(cur);
  if (st != MK_OK) return st;
  *stale = *timeouts = 0;
  for (int p = 0; p < pairs; ++p) {
    *stale += res[2 * p];
    *timeouts += res[2 * p + 1];
  }
  return MK_OK;
}

mk_status mk_kv_cache(mk_handle* h, int layer, void** kv_base, size_t* bytes) {
  if (!h || !kv_base || !bytes) return MK_ERR_INVALID_ARG;
  if (h->host_only) return fail(h, MK_ERR_STATE, "host-only handle");
  if (layer < 0 || layer >= h->cfg.n_layers) return fail(h, MK_ERR_INVALID_ARG, "layer %d out of range", layer);
  const size_t per = h->kv_bytes / h->cfg.n_layers;
  *kv_base = (char*)h->kv + per * layer;
  *bytes = per;
  return MK_OK;
}

mk_status mk_set_routing_trace(mk_handle* h, int32_t* trace) {
  if (!h) return MK_ERR_INVALID_ARG;
  h->tk_trace = trace;
  return MK_OK;
}

mk_status mk_sync_status(mk_handle* h, void* stream) {
  if (!h) return MK_ERR_INVALID_ARG;
  if (h->host_only) return MK_OK;
  HIPCHECK(h, hipSetDevice(h->device));
  HIPCHECK(h, hipStreamSynchronize((hipStream_t)stream));
  uint32_t e[4];
  HIPCHECK(h, hipMemcpy(e, h->err_word, sizeof(e), hipMemcpyDeviceToHost));
  if (e[0] == 0 && h->static_used) {
    // the allocation-free step's error word (in this device's static array)
    uint32_t* se = (uint32_t*)((char*)h->static_scratch + h->lay.err);
    HIPCHECK(h, hipMemcpy(e, se, sizeof(e), hipMemcpyDeviceToHost));
    if (e[0] != 0) HIPCHECK(h, hipMemset(se, 0, sizeof(e)));
  }
  if (e[0] == 0) return MK_OK;
  HIPCHECK(h, hipMemset(h->err_word, 0, sizeof(e)));
  // a failed step leaves counters mid-way: clear both sets
  for (auto* c : h->ctr) HIPCHECK(h, hipMemset(c, 0, (size_t)h->n_ctr_cap * 4));
  HIPCHECK(h, hipDeviceSynchronize());
  if (e[0] == MK_DEVERR_TIMEOUT)
    return fail(h, MK_ERR_DEVICE_TIMEOUT, "device wait timed out on counter %u (value %u, workgroup %u)", e[1], e[2],
                e[3]);
  return fail(h, MK_ERR_DEVICE_FAULT, "device rejected an index (site %u, value %u, workgroup %u)", e[1], e[2], e[3]);
}

mk_status mk_debug_read(mk_handle* h, const char* name, void* host, size_t bytes) {
  if (!h || !name || !host) return MK_ERR_INVALID_ARG;
  if (h->host_only) return fail(h, MK_ERR_STATE, "host-only handle");
  const mk_config& c = h->cfg;
  const size_t Bm = c.max_batch, H = c.hidden, E = c.n_experts, K = c.top_k;
  struct Item { const char* n; const void* p; size_t sz; };
  const Item items[] = {
      {"h", h->h, Bm * H * 4},
      {"ssq", h->ssq, 2 * Bm * h->NB * 4},
      {"u", h->u, 4 * Bm * H * 2},
      {"q", h->q, Bm * h->q_dim * 4},
      {"o", h->o, 2 * Bm * h->q_dim * 2},
      {"ao", h->ao, (size_t)c.n_kv_heads * Bm * H * 4},
      {"rp", h->rp, (size_t)h->router_ks * Bm * E * 4},
      {"tk_idx", h->tk_idx, Bm * K * 4},
      {"tk_w", h->tk_w, Bm * K * 4},
      {"route", h->route, (size_t)MK_ROUTE_INTS(E, Bm) * 4},
      {"gu", h->gu, Bm * K * 4 * c.expert_ffn * 4},
      {"dn", h->dn, Bm * K * H * 4},
      {"mp", h->mp, (size_t)std::max(h->n_workers, 1) * MK_FUSED_B * H * 4},
  };
  for (const Item& it : items)
    if (std::strcmp(it.n, name) == 0) {
      if (bytes > it.sz) return fail(h, MK_ERR_INVALID_ARG, "%s holds %zu bytes", name, it.sz);
      HIPCHECK(h, hipSetDevice(h->device));
      HIPCHECK(h, hipDeviceSynchronize());
      if (std::strcmp(name, "q") == 0 && h->last_tagged) {
        // the last step handed the queries over as tagged words: their values
        const size_t rows = std::min<size_t>(Bm, MK_FUSED_B), n = rows * h->q_dim;
        std::vector<uint64_t> w(n);
        HIPCHECK(h, hipMemcpy(w.data(), h->qt, n * 8, hipMemcpyDeviceToHost));
        std::memset(host, 0, bytes);
        uint32_t* dst = (uint32_t*)host;
        for (size_t i = 0; i < n && i < bytes / 4; ++i) dst[i] = (uint32_t)w[i];
        return MK_OK;
      }
      HIPCHECK(h, hipMemcpy(host, it.p, bytes, hipMemcpyDeviceToHost));
      return MK_OK;
    }
  return fail(h, MK_ERR_INVALID_ARG, "unknown scratch buffer '%s'", name);
}

mk_status mk_schedule_info_get(mk_handle* h, int batch, int hint, mk_schedule_info* out) {
  if (!h || !out) return MK_ERR_INVALID_ARG;
  if (batch < 1 || batch > h->cfg.max_batch || hint < 1 || hint > h->cfg.max_seq_len)
    return fail(h, MK_ERR_INVALID_ARG, "bad batch/hint");
  Schedule* S = nullptr;
  mk_status st = get_schedule(h, batch, hint, &S);
  if (st != MK_OK) return st;
  out->n_tasks = (int32_t)S->cu_tasks.size();
  int mx = 0;
  for (int i = 0; i < h->n_workers; ++i) mx = std::max(mx, S->cu_off[i + 1] - S->cu_off[i]);
  out->max_tasks_per_cu = mx;
  out->n_counters = S->n_ctr;
  out->n_cus = h->n_workers;
  const mk_config& c = h->cfg;
  const int64_t per_layer = (int64_t)c.hidden * h->qkv_dim + (int64_t)h->q_dim * c.hidden +
                            (int64_t)c.hidden * h->e_pad + c.hidden +
                            (int64_t)c.top_k * 3 * c.hidden * c.expert_ffn;
  out->weight_bytes_per_step = 2 * (per_layer * c.n_layers + (int64_t)c.hidden * c.vocab + c.hidden);
  return MK_OK;
}

mk_status mk_schedule_export(mk_handle* h, int batch, int hint, int32_t* tasks, int32_t* cu_offsets) {
  if (!h || !tasks || !cu_offsets) return MK_ERR_INVALID_ARG;
  Schedule* S = nullptr;
  mk_status st = get_schedule(h, batch, hint, &S);
  if (st != MK_OK) return st;
  std::memcpy(tasks, S->cu_tasks.data(), S->cu_tasks.size() * sizeof(mk_task));
  std::memcpy(cu_offsets, S->cu_off.data(), S->cu_off.size() * sizeof(int32_t));
  return MK_OK;
}

mk_status mk_schedule_check(mk_handle* h, int batch, int hint, uint32_t flags, char* report, size_t report_len) {
  if (!h) return MK_ERR_INVALID_ARG;
  if (batch < 1 || batch > h->cfg.max_batch || hint < 1 || hint > h->cfg.max_seq_len)
    return fail(h, MK_ERR_INVALID_ARG, "bad batch/hint");
  Schedule* S = nullptr;
  mk_status st = get_schedule(h, batch, hint, &S);
  if (st != MK_OK) return st;
  std::string rep;
  st = check_hazards(h, *S, flags, rep);
  if (report && report_len) {
    std::strncpy(report, rep.c_str(), report_len - 1);
    report[report_len - 1] = 0;
  }
  return st;
}

mk_status mk_schedule_simulate(mk_handle* h, int batch, int hint, const int32_t* n_active, uint64_t seed,
                               int32_t corrupt_task, char* report, size_t report_len) {
  if (!h || !n_active) return MK_ERR_INVALID_ARG;
  if (batch < 1 || batch > h->cfg.max_batch || hint < 1 || hint > h->cfg.max_seq_len)
    return fail(h, MK_ERR_INVALID_ARG, "bad batch/hint");
  for (int l = 0; l < h->cfg.n_layers; ++l)
    if (n_active[l] < 1 || n_active[l] > std::min(h->cfg.n_experts, batch * h->cfg.top_k))
      return fail(h, MK_ERR_INVALID_ARG, "n_active[%d] out of range", l);
  Schedule* S = nullptr;
  mk_status st = get_schedule(h, batch, hint, &S);
  if (st != MK_OK) return st;
  std::string rep;
  st = simulate(h, *S, n_active, seed, corrupt_task, rep);
  if (report && report_len) {
    std::strncpy(report, rep.c_str(), report_len - 1);
    report[report_len - 1] = 0;
  }
  return st;
}

}  // extern "C"
