// mk_service.cpp - the host decode service around mk_decode_step.
//
// Cohere's North Mini Code megakernel post (Chinese version, section on the
// inference engine around the kernel, "Python and C++ take turns") runs two
// long-lived host threads: a control plane that receives requests, prefills
// them and manages KV capacity and the batch, and a native thread that only
// decodes. The control plane pauses the decoder to change the batch; the
// decoder finishes its current step, parks (the GPU idle, batch state no
// longer read), and after the resume snapshots the new batch and keeps
// decoding. Its loop per step: update the KV page tables, clear scratch and
// barriers, select the schedule for the longest live context, launch the
// megakernel, sample and stream the tokens, retire finished requests.
//
// Here the decoding thread is a std::thread per service. Clearing scratch and
// barriers happens inside the kernel (each step clears the next step's
// counters); the schedule is selected by mk_decode_step from the batch size
// and the longest context; sampling is the kernel's greedy token. Pages come
// from a free list the service owns: the control plane takes pages from it to
// hold a request's context (written through mk_kv_cache while parked), the
// decoder adds one whenever a sequence crosses into a new page, and a retired
// or evicted request's pages return to it.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <condition_variable>
#include <cstring>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "../../include/mk.h"
#include "mk_internal.h"

namespace {

struct Seq {
  int64_t id;
  int32_t token;       // the token to decode next
  int32_t len;         // positions in the cache after this step's append (context + decoded + 1)
  int32_t generated;   // tokens streamed so far
  int32_t max_new;
  int32_t stop_token;  // -1: none
  std::vector<int32_t> pages;
};

}  // namespace

struct mk_service {
  mk_handle* h = nullptr;
  mk_service_config cfg{};
  int page_size = 16, mpps = 0, vocab = 0;
  hipStream_t stream = nullptr;
  bool own_stream = false;
  // device batch arrays and pinned host mirrors
  int32_t *d_tokens = nullptr, *d_lens = nullptr, *d_bt = nullptr, *d_next = nullptr;
  float* d_logits = nullptr;
  int32_t *p_tokens = nullptr, *p_lens = nullptr, *p_bt = nullptr, *p_next = nullptr;
  // state (mu guards everything below)
  std::mutex mu;
  std::condition_variable cv;
  std::vector<Seq> active;
  std::vector<int32_t> free_pages;
  bool pause_req = false, parked = false, stop = false;
  mk_status failure = MK_OK;
  std::string err;
  int64_t steps = 0, tokens = 0;
  std::thread th;

  void loop();
};

namespace {

mk_status svc_fail(mk_service* s, mk_status st, const char* msg) {
  s->err = msg;
  return st;
}

}  // namespace

void mk_service::loop() {
  std::unique_lock<std::mutex> lk(mu);
  for (;;) {
    if (stop) break;
    if (pause_req || active.empty() || failure != MK_OK) {
      parked = true;
      cv.notify_all();
      cv.wait(lk, [&] { return stop || (!pause_req && !active.empty() && failure == MK_OK); });
      parked = false;
      continue;
    }
    // update the page tables: a sequence whose next position starts a page
    // gets one from the free list (none left: the request fails)
    const int B = (int)active.size();
    int max_len = 0;
    for (int b = 0; b < B; ++b) {
      Seq& q = active[b];
      const int need = (q.len + page_size - 1) / page_size;
      while ((int)q.pages.size() < need) {
        if (free_pages.empty() || (int)q.pages.size() >= mpps) {
          failure = MK_ERR_OOM;
          err = "decode service: no free KV page for a growing sequence";
          break;
        }
        q.pages.push_back(free_pages.back());
        free_pages.pop_back();
      }
      if (failure != MK_OK) break;
      p_tokens[b] = q.token;
      p_lens[b] = q.len;
      for (int j = 0; j < mpps; ++j) p_bt[b * mpps + j] = j < (int)q.pages.size() ? q.pages[j] : -1;
      max_len = std::max(max_len, q.len);
    }
    if (failure != MK_OK) continue;
    // the step runs without the lock: the control plane only changes the
    // batch while the loop is parked
    lk.unlock();
    mk_status st = MK_OK;
    hipError_t e = hipMemcpyAsync(d_tokens, p_tokens, B * 4, hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipMemcpyAsync(d_lens, p_lens, B * 4, hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipMemcpyAsync(d_bt, p_bt, (size_t)B * mpps * 4, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) st = MK_ERR_HIP;
    if (st == MK_OK)
      st = mk_decode_step(h, B, d_tokens, d_bt, d_lens, max_len, d_logits, d_next, 0, stream);
    if (st == MK_OK && hipMemcpyAsync(p_next, d_next, B * 4, hipMemcpyDeviceToHost, stream) != hipSuccess)
      st = MK_ERR_HIP;
    if (st == MK_OK) st = mk_sync_status(h, stream);  // synchronises the stream
    lk.lock();
    if (st != MK_OK) {
      failure = st;
      err = std::string("decode service step failed: ") + mk_last_error(h);
      for (const Seq& q : active)
        if (cfg.on_token) cfg.on_token(cfg.user, q.id, -1, -1);
      continue;
    }
    ++steps;
    // stream the tokens, retire finished requests (their pages return)
    std::vector<Seq> keep;
    keep.reserve(active.size());
    for (int b = 0; b < B; ++b) {
      Seq& q = active[b];
      const int32_t tok = p_next[b];
      ++q.generated;
      ++tokens;
      const bool done = q.generated >= q.max_new || tok == q.stop_token;
      if (cfg.on_token) cfg.on_token(cfg.user, q.id, tok, done ? 1 : 0);
      if (done) {
        free_pages.insert(free_pages.end(), q.pages.begin(), q.pages.end());
      } else {
        q.token = tok;
        q.len += 1;
        keep.push_back(std::move(q));
      }
    }
    active.swap(keep);
  }
  parked = true;
  cv.notify_all();
}

extern "C" {

mk_status mk_service_create(mk_handle* h, const mk_service_config* cfg, mk_service** out) {
  if (!h || !cfg || !out) return MK_ERR_INVALID_ARG;
  *out = nullptr;
  int max_batch = 0, mpps = 0, n_pages = 0, vocab = 0;
  if (!mk_handle_dims(h, &max_batch, &mpps, &n_pages, &vocab)) return MK_ERR_STATE;
  if (cfg->max_batch < 1 || cfg->max_batch > max_batch) return MK_ERR_INVALID_ARG;
  if (cfg->page0 < 0 || cfg->n_pages < 1 || cfg->page0 + cfg->n_pages > n_pages) return MK_ERR_INVALID_ARG;
  auto s = new mk_service();
  s->h = h;
  s->cfg = *cfg;
  s->mpps = mpps;
  s->vocab = vocab;
  for (int p = cfg->page0 + cfg->n_pages - 1; p >= cfg->page0; --p) s->free_pages.push_back(p);
  bool ok = true;
  if (cfg->stream) {
    s->stream = (hipStream_t)cfg->stream;
  } else {
    ok = hipStreamCreate(&s->stream) == hipSuccess;
    s->own_stream = ok;
  }
  const int Bm = cfg->max_batch;
  ok = ok && hipMalloc(&s->d_tokens, Bm * 4) == hipSuccess && hipMalloc(&s->d_lens, Bm * 4) == hipSuccess &&
       hipMalloc(&s->d_next, Bm * 4) == hipSuccess && hipMalloc(&s->d_bt, (size_t)Bm * mpps * 4) == hipSuccess &&
       hipMalloc(&s->d_logits, (size_t)Bm * vocab * 4) == hipSuccess;
  ok = ok && hipHostMalloc(&s->p_tokens, Bm * 4) == hipSuccess && hipHostMalloc(&s->p_lens, Bm * 4) == hipSuccess &&
       hipHostMalloc(&s->p_next, Bm * 4) == hipSuccess &&
       hipHostMalloc(&s->p_bt, (size_t)Bm * mpps * 4) == hipSuccess;
  if (!ok) {
    mk_service_destroy(s);
    return MK_ERR_OOM;
  }
  // start paused: the control plane admits requests, then resumes
  s->pause_req = true;
  s->th = std::thread([s] { s->loop(); });
  {
    std::unique_lock<std::mutex> lk(s->mu);
    s->cv.wait(lk, [&] { return s->parked; });
  }
  *out = s;
  return MK_OK;
}

mk_status mk_service_pause(mk_service* s) {
  if (!s) return MK_ERR_INVALID_ARG;
  std::unique_lock<std::mutex> lk(s->mu);
  s->pause_req = true;
  s->cv.notify_all();
  s->cv.wait(lk, [&] { return s->parked; });
  return MK_OK;
}

mk_status mk_service_resume(mk_service* s) {
  if (!s) return MK_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(s->mu);
  s->pause_req = false;
  s->cv.notify_all();
  return MK_OK;
}

mk_status mk_service_alloc_pages(mk_service* s, int32_t n, int32_t* pages) {
  if (!s || n < 0 || (n > 0 && !pages)) return MK_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(s->mu);
  if (!s->parked || !s->pause_req) return svc_fail(s, MK_ERR_STATE, "pages are handed out while the service is paused");
  if ((int)s->free_pages.size() < n) return svc_fail(s, MK_ERR_OOM, "not enough free KV pages");
  for (int i = 0; i < n; ++i) {
    pages[i] = s->free_pages.back();
    s->free_pages.pop_back();
  }
  return MK_OK;
}

mk_status mk_service_admit(mk_service* s, int64_t request_id, int32_t first_token, int32_t context_len,
                           const int32_t* pages, int32_t n_pages, int32_t max_new_tokens, int32_t stop_token) {
  if (!s) return MK_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(s->mu);
  if (!s->parked || !s->pause_req) return svc_fail(s, MK_ERR_STATE, "requests are admitted while the service is paused");
  if ((int)s->active.size() >= s->cfg.max_batch) return svc_fail(s, MK_ERR_UNSUPPORTED, "the batch is full");
  if (first_token < 0 || first_token >= s->vocab || context_len < 0 || max_new_tokens < 1 || n_pages < 0 ||
      (n_pages > 0 && !pages) || n_pages * s->page_size < context_len || n_pages > s->mpps)
    return svc_fail(s, MK_ERR_INVALID_ARG, "bad request");
  for (const Seq& q : s->active)
    if (q.id == request_id) return svc_fail(s, MK_ERR_INVALID_ARG, "request id already active");
  Seq q;
  q.id = request_id;
  q.token = first_token;
  q.len = context_len + 1;
  q.generated = 0;
  q.max_new = max_new_tokens;
  q.stop_token = stop_token;
  q.pages.assign(pages, pages + n_pages);
  s->active.push_back(std::move(q));
  return MK_OK;
}

mk_status mk_service_evict(mk_service* s, int64_t request_id) {
  if (!s) return MK_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(s->mu);
  if (!s->parked || !s->pause_req) return svc_fail(s, MK_ERR_STATE, "requests are evicted while the service is paused");
  for (size_t i = 0; i < s->active.size(); ++i)
    if (s->active[i].id == request_id) {
      s->free_pages.insert(s->free_pages.end(), s->active[i].pages.begin(), s->active[i].pages.end());
      s->active.erase(s->active.begin() + i);
      return MK_OK;
    }
  return svc_fail(s, MK_ERR_INVALID_ARG, "no such request");
}

mk_status mk_service_stats(mk_service* s, mk_service_info* out) {
  if (!s || !out) return MK_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(s->mu);
  out->steps = s->steps;
  out->tokens = s->tokens;
  out->active = (int32_t)s->active.size();
  out->free_pages = (int32_t)s->free_pages.size();
  out->parked = s->parked ? 1 : 0;
  out->status = s->failure;
  return MK_OK;
}

const char* mk_service_last_error(const mk_service* s) { return s ? s->err.c_str() : ""; }

void mk_service_destroy(mk_service* s) {
  if (!s) return;
  {
    std::lock_guard<std::mutex> lk(s->mu);
    s->stop = true;
    s->cv.notify_all();
  }
  if (s->th.joinable()) s->th.join();
  hipFree(s->d_tokens);
  hipFree(s->d_lens);
  hipFree(s->d_next);
  hipFree(s->d_bt);
  hipFree(s->d_logits);
  hipHostFree(s->p_tokens);
  hipHostFree(s->p_lens);
  hipHostFree(s->p_next);
  hipHostFree(s->p_bt);
  if (s->own_stream) hipStreamDestroy(s->stream);
  delete s;
}

}  // extern "C"
