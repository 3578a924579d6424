// The serving loop's decode owner: a C++ thread that owns an engine and runs decode steps over a
// continuously changing batch (P3 "Scheduling and Performance Benchmarks": a C++ thread owns the
// decode loop while the control side - requests, prefill, batch management - runs in Python; P1
// "From demo to a full serving system": continuous batching with ragged lengths).
//
// A sequence arrives either with its prefill done elsewhere (its K/V for positions [0, prompt_len)
// already in the pages it owns) or with its prompt tokens, which the owner then prefills itself:
// every step, each decoding sequence takes one batch row and the rows left over go to prompt chunks
// (consecutive positions of one sequence, one per row), so prefill and decode share steps (P3
// "Limitations and Future Plans": mixed batches are the pages' next step). Sequences are admitted at
// step boundaries while fewer than max_batch are active; a sequence leaves once it has generated its
// budget of tokens. Whenever the rows' composition changes, the block tables are re-uploaded and the
// schedule rebuilt. The control side can pause decode between steps (for a prefill it runs itself on
// the same GPU, as the pages do) and can give the owner a step budget (manual stepping, used by the
// tests).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <condition_variable>
#include <cstdio>
#include <cstring>
#include <deque>
#include <map>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "../../include/mk.h"
#include "mk_internal.h"
#include "mk_launch.h"

namespace {

struct Seq {
  int64_t id = -1;
  int32_t pos = 0;               // next position: a prompt chunk's first row while pos < decode_at
  int32_t decode_at = 0;         // position of the first decoded token (prompt positions lie before it)
  int32_t token = 0;             // token decoded at decode_at (and later the last generated one)
  int32_t remaining = 0;         // tokens still to generate
  std::vector<int32_t> prompt;   // prompt tokens still to prefill are prompt[pos] .. prompt[decode_at - 1]
  std::vector<int32_t> pages;
  std::vector<int32_t> out;      // generated tokens
  bool prefilling() const { return pos < decode_at; }
};

struct Row {                     // one batch row of a step
  int seq;                       // index into the step's active list
  int32_t pos, token;
};

}  // namespace

struct mk_server {
  mk_engine* e = nullptr;
  mk_model_desc desc{};
  int max_batch = 0;
  int device = 0;
  hipStream_t stream = nullptr;
  // device buffers for the step's inputs and outputs (allocated at create, never per step)
  int32_t *d_tokens = nullptr, *d_pos = nullptr, *d_lens = nullptr, *d_bt = nullptr, *d_argmax = nullptr;
  float* d_logits = nullptr;
  // pinned host staging for the per-step copies
  int32_t* h_in = nullptr;        // [3][max_batch]: tokens, positions, seq_lens
  int32_t* h_argmax = nullptr;    // [max_batch]
  // optional per-step outputs of the caller (device pointers, set at create)
  int32_t* topk_out = nullptr;
  float* rlog_out = nullptr;
  float* hidden_out = nullptr;
  float* logits_out = nullptr;    // caller-owned [max_batch, vocab] logits (NULL: the server's own)

  std::mutex mu;
  std::condition_variable cv;     // the owner waits for work; waiters wait for the owner
  std::thread owner;
  bool stop = false, pause_req = false, paused = false, busy = false;
  int64_t budget = -1;            // steps still allowed (-1: no limit)
  std::deque<Seq> pending;        // admitted at the next step boundary
  std::vector<Seq> rows;          // active sequences (admission order)
  std::vector<Seq> done;          // finished, not yet collected
  int64_t steps = 0, tokens = 0, rebuilds = 0, prefill_tokens = 0;
  double busy_s = 0;
  mk_status status = MK_OK;       // first failure of the owner (sticky)
  std::string msg;
  mk_server_step last{};          // composition of the last step
};

namespace {

void fail(mk_server* s, mk_status st, const std::string& what) {
  if (s->status == MK_OK) {
    s->status = st;
    char buf[512];
    buf[0] = 0;
    if (s->e) mk_get_error(s->e, buf, sizeof buf);
    s->msg = what + (buf[0] ? std::string(": ") + buf : std::string());
  }
}

// The step's rows: one per decoding sequence, then the rows left over as prompt chunks, in admission
// order (owner thread). `key` (sequence id and row count per sequence) identifies the composition.
std::vector<Row> compose(const std::vector<Seq>& act, int max_batch, std::vector<int64_t>* key, int* rows_per_seq) {
  std::vector<Row> rows;
  std::vector<int> cnt(act.size(), 0);
  for (int i = 0; i < (int)act.size(); ++i)
    if (!act[i].prefilling()) { rows.push_back({i, act[i].pos, act[i].token}); cnt[i] = 1; }
  for (int i = 0; i < (int)act.size() && (int)rows.size() < max_batch; ++i) {
    const Seq& q = act[i];
    if (!q.prefilling()) continue;
    const int c = std::min(max_batch - (int)rows.size(), q.decode_at - q.pos);
    for (int r = 0; r < c; ++r) rows.push_back({i, q.pos + r, q.prompt[q.pos + r]});
    cnt[i] = c;
  }
  key->clear();
  *rows_per_seq = 1;
  for (int i = 0; i < (int)act.size(); ++i) {
    key->push_back(act[i].id);
    key->push_back(cnt[i]);
    *rows_per_seq = std::max(*rows_per_seq, cnt[i]);
  }
  return rows;
}

// Upload the rows' block tables and rebuild the schedule (owner thread, unlocked).
mk_status rebuild(mk_server* s, const std::vector<Seq>& act, const std::vector<Row>& rows, int rows_per_seq) {
  const int B = (int)rows.size(), P = s->desc.max_pages_per_seq;
  std::vector<int32_t> bt((size_t)s->max_batch * P, -1), lens(B);
  for (int b = 0; b < B; ++b) {
    const Seq& q = act[rows[b].seq];
    std::copy(q.pages.begin(), q.pages.end(), bt.begin() + (size_t)b * P);
    lens[b] = rows[b].pos + 1;
  }
  if (hipMemcpyAsync(s->d_bt, bt.data(), bt.size() * sizeof(int32_t), hipMemcpyHostToDevice, s->stream) != hipSuccess ||
      hipStreamSynchronize(s->stream) != hipSuccess)
    return MK_ERR_HIP;
  return mk_build_schedule_chunked(s->e, B, lens.data(), rows_per_seq);
}

// Keys a row may grow past the length its schedule was built for before the owner rebuilds it: half
// an attention split (the open-ended last split takes every new key and lies on the critical path;
// the owner already rebuilds at every change of the batch, so a longer interval than the engine's
// quarter split keeps the host's share of the step down: measured 226 generated tok/s at half a
// split, 221 at a quarter)
int refresh_keys(mk_server* s) {
  mk_plan_info info{};
  if (mk_plan_info_get(mk_engine_plan(s->e), &info) != MK_OK || info.split_keys < 2) return 1 << 30;
  return info.split_keys / 2;
}

void owner_loop(mk_server* s) {
  (void)hipSetDevice(s->device);
  std::unique_lock<std::mutex> lk(s->mu);
  std::vector<int64_t> built_key;               // composition the current schedule was built for
  std::vector<int> built_len;                   // and each row's length then
  int refresh = 1 << 30;
  bool have_schedule = false;
  for (;;) {
    s->cv.wait(lk, [&] {
      if (s->stop || s->pause_req) return true;
      if (s->status != MK_OK || s->budget == 0) return false;
      const bool admit = !s->pending.empty() && (int)s->rows.size() < s->max_batch;
      return admit || !s->rows.empty();
    });
    if (s->stop) break;
    if (s->pause_req) {                       // decode paused: a prefill may use the GPU now
      s->paused = true;
      s->cv.notify_all();
      s->cv.wait(lk, [&] { return s->stop || !s->pause_req; });
      s->paused = false;
      continue;
    }
    while (!s->pending.empty() && (int)s->rows.size() < s->max_batch) {
      s->rows.push_back(std::move(s->pending.front()));
      s->pending.pop_front();
    }
    std::vector<Seq> act = s->rows;           // the owner's working copy for this step
    s->busy = true;
    lk.unlock();

    const auto t0 = std::chrono::steady_clock::now();
    std::vector<int64_t> key;
    int rows_per_seq = 1;
    const std::vector<Row> rows = compose(act, s->max_batch, &key, &rows_per_seq);
    const int B = (int)rows.size();
    mk_status st = MK_OK;
    std::string what;
    bool changed = !have_schedule || key != built_key || (int)built_len.size() != B;
    for (int b = 0; b < B && !changed; ++b) changed = rows[b].pos + 1 - built_len[b] >= refresh;
    if (changed) {
      st = rebuild(s, act, rows, rows_per_seq);
      what = "mk_build_schedule";
      have_schedule = st == MK_OK;
      built_key = key;
      built_len.resize(B);
      for (int b = 0; b < B; ++b) built_len[b] = rows[b].pos + 1;
      if (have_schedule) refresh = refresh_keys(s);
    }
    for (int b = 0; b < B && st == MK_OK; ++b) {
      s->h_in[b] = rows[b].token;
      s->h_in[s->max_batch + b] = rows[b].pos;
      s->h_in[2 * s->max_batch + b] = rows[b].pos + 1;
    }
    if (st == MK_OK &&
        (hipMemcpyAsync(s->d_tokens, s->h_in, B * sizeof(int32_t), hipMemcpyHostToDevice, s->stream) != hipSuccess ||
         hipMemcpyAsync(s->d_pos, s->h_in + s->max_batch, B * sizeof(int32_t), hipMemcpyHostToDevice, s->stream) != hipSuccess ||
         hipMemcpyAsync(s->d_lens, s->h_in + 2 * s->max_batch, B * sizeof(int32_t), hipMemcpyHostToDevice, s->stream) != hipSuccess)) {
      st = MK_ERR_HIP;
      what = "copying the step's inputs";
    }
    bool rebuilt = changed && st == MK_OK;
    if (st == MK_OK) {
      float* L = s->logits_out ? s->logits_out : s->d_logits;
      st = mk_decode_step(s->e, s->d_tokens, s->d_pos, s->d_bt, s->d_lens, L, s->stream);
      if (st == MK_ERR_SCHEDULE_STALE) {      // a sequence outgrew its attention splits: rebuild, retry
        st = rebuild(s, act, rows, rows_per_seq);
        rebuilt = st == MK_OK;
        built_len.resize(B);
        for (int b = 0; b < B; ++b) built_len[b] = rows[b].pos + 1;
        if (st == MK_OK) st = mk_decode_step(s->e, s->d_tokens, s->d_pos, s->d_bt, s->d_lens, L, s->stream);
      }
      what = "mk_decode_step";
    }
    if (st == MK_OK && (hipMemcpyAsync(s->h_argmax, s->d_argmax, B * sizeof(int32_t), hipMemcpyDeviceToHost, s->stream) != hipSuccess ||
                        hipStreamSynchronize(s->stream) != hipSuccess)) {
      st = MK_ERR_HIP;
      what = "reading the step's tokens";
    }
    if (st == MK_OK) {
      st = mk_sync(s->e);
      what = "the step kernel";
    }
    const double dt = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();

    lk.lock();
    s->busy = false;
    if (st != MK_OK) {
      fail(s, st, what);
      s->cv.notify_all();
      continue;                               // the owner idles until destroyed
    }
    if (rebuilt) s->rebuilds++;
    mk_server_step& rec = s->last;
    rec.step = s->steps;
    rec.batch = B;
    int n_prefill = 0;
    for (int b = 0; b < MK_MAX_BATCH; ++b) {
      const bool pf = b < B && rows[b].pos < act[rows[b].seq].decode_at;
      n_prefill += pf ? 1 : 0;
      rec.request_id[b] = b < B ? act[rows[b].seq].id : -1;
      rec.position[b] = b < B ? rows[b].pos : -1;
      rec.token_in[b] = b < B ? rows[b].token : -1;
      rec.token_out[b] = b < B && !pf ? s->h_argmax[b] : -1;   // prompt rows generate nothing
    }
    rec.rebuilt = rebuilt ? 1 : 0;
    rec.prefill_rows = n_prefill;
    // advance every sequence (the active list only grew at the back since the step began); finished
    // sequences leave the batch
    std::vector<int> adv(act.size(), 0);
    for (int b = 0; b < B; ++b) {
      Seq& q = s->rows[rows[b].seq];
      if (rows[b].pos < act[rows[b].seq].decode_at) { adv[rows[b].seq]++; continue; }
      q.out.push_back(s->h_argmax[b]);
      q.token = s->h_argmax[b];
      q.pos += 1;
      q.remaining -= 1;
    }
    for (int i = 0; i < (int)act.size(); ++i) s->rows[i].pos += adv[i];
    std::vector<Seq> keep;
    for (auto& q : s->rows) {
      if (q.remaining <= 0) s->done.push_back(std::move(q));
      else keep.push_back(std::move(q));
    }
    s->rows = std::move(keep);
    s->steps++;
    s->tokens += B - n_prefill;
    s->prefill_tokens += n_prefill;
    s->busy_s += dt;
    if (s->budget > 0) s->budget--;
    s->cv.notify_all();
  }
  s->cv.notify_all();
}

}  // namespace

extern "C" {

mk_status mk_server_create(mk_engine* e, const mk_server_config* cfg, mk_server** out) {
  if (!e || !cfg || !out) return MK_ERR_INVALID_ARG;
  *out = nullptr;
  const mk_model_desc& d = engine_desc(e);
  if (cfg->max_batch < 1 || cfg->max_batch > d.max_batch) return MK_ERR_INVALID_ARG;
  mk_server* s = new mk_server();
  s->e = e;
  s->desc = d;
  s->max_batch = cfg->max_batch;
  s->budget = cfg->start_held ? 0 : -1;
  s->topk_out = cfg->topk_out;
  s->logits_out = cfg->logits_out;
  s->rlog_out = cfg->router_logits_out;
  s->hidden_out = cfg->hidden_out;
  const int B = s->max_batch;
  auto cleanup = [&](mk_status st) {
    void* dp[] = {s->d_tokens, s->d_pos, s->d_lens, s->d_bt, s->d_argmax, s->d_logits};
    for (void* p : dp) if (p) (void)hipFree(p);
    if (s->h_in) (void)hipHostFree(s->h_in);
    if (s->h_argmax) (void)hipHostFree(s->h_argmax);
    if (s->stream) (void)hipStreamDestroy(s->stream);
    delete s;
    return st;
  };
  if (hipGetDevice(&s->device) != hipSuccess || hipStreamCreate(&s->stream) != hipSuccess) return cleanup(MK_ERR_HIP);
  const size_t V = (size_t)std::max(d.vocab, 1);
  if (hipMalloc(&s->d_tokens, B * sizeof(int32_t)) != hipSuccess || hipMalloc(&s->d_pos, B * sizeof(int32_t)) != hipSuccess ||
      hipMalloc(&s->d_lens, B * sizeof(int32_t)) != hipSuccess || hipMalloc(&s->d_argmax, B * sizeof(int32_t)) != hipSuccess ||
      hipMalloc(&s->d_bt, (size_t)B * d.max_pages_per_seq * sizeof(int32_t)) != hipSuccess ||
      (!s->logits_out && hipMalloc(&s->d_logits, (size_t)B * V * sizeof(float)) != hipSuccess) ||
      hipHostMalloc((void**)&s->h_in, 3 * B * sizeof(int32_t), hipHostMallocDefault) != hipSuccess ||
      hipHostMalloc((void**)&s->h_argmax, B * sizeof(int32_t), hipHostMallocDefault) != hipSuccess)
    return cleanup(MK_ERR_OOM);
  if (hipMemset(s->d_argmax, 0, B * sizeof(int32_t)) != hipSuccess) return cleanup(MK_ERR_HIP);
  if (s->logits_out) s->d_logits = nullptr;
  const mk_status st = mk_set_step_outputs(e, s->d_argmax, s->topk_out, s->hidden_out, nullptr, s->rlog_out);
  if (st != MK_OK) return cleanup(st);
  s->owner = std::thread(owner_loop, s);
  *out = s;
  return MK_OK;
}

mk_status mk_server_submit(mk_server* s, const mk_request* r) {
  if (!s || !r || r->prompt_len < 0 || r->max_new_tokens < 1 || r->n_pages < 1 || !r->pages)
    return MK_ERR_INVALID_ARG;
  Seq q;
  if (r->prompt) {                      // the owner prefills positions [0, prompt_len - 1)
    if (r->prompt_len < 1) return MK_ERR_INVALID_ARG;
    for (int i = 0; i < r->prompt_len; ++i)
      if (r->prompt[i] < 0 || r->prompt[i] >= s->desc.vocab) return MK_ERR_INVALID_ARG;
    q.prompt.assign(r->prompt, r->prompt + r->prompt_len);
    q.pos = 0;
    q.decode_at = r->prompt_len - 1;
    q.token = r->prompt[r->prompt_len - 1];
  } else {
    if (r->first_token < 0 || r->first_token >= s->desc.vocab) return MK_ERR_INVALID_ARG;
    q.pos = q.decode_at = r->prompt_len;
    q.token = r->first_token;
  }
  const int64_t need = (int64_t)q.decode_at + r->max_new_tokens;     // positions the sequence will hold
  if (r->n_pages > s->desc.max_pages_per_seq || need > (int64_t)r->n_pages * mk::PAGE) return MK_ERR_INVALID_ARG;
  for (int i = 0; i < r->n_pages; ++i)
    if (r->pages[i] < 0 || r->pages[i] >= s->desc.num_pages) return MK_ERR_INVALID_ARG;
  q.id = r->request_id;
  q.remaining = r->max_new_tokens;
  q.pages.assign(r->pages, r->pages + r->n_pages);
  std::lock_guard<std::mutex> lk(s->mu);
  if (s->status != MK_OK) return s->status;
  s->pending.push_back(std::move(q));
  s->cv.notify_all();
  return MK_OK;
}

mk_status mk_server_pause(mk_server* s) {
  if (!s) return MK_ERR_INVALID_ARG;
  std::unique_lock<std::mutex> lk(s->mu);
  s->pause_req = true;
  s->cv.notify_all();
  s->cv.wait(lk, [&] { return s->paused || s->status != MK_OK; });
  return s->status;
}

mk_status mk_server_resume(mk_server* s) {
  if (!s) return MK_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(s->mu);
  s->pause_req = false;
  s->cv.notify_all();
  return s->status;
}

mk_status mk_server_run(mk_server* s, int64_t n_steps) {
  if (!s || n_steps < -1) return MK_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(s->mu);
  s->budget = n_steps;
  s->cv.notify_all();
  return s->status;
}

mk_status mk_server_wait(mk_server* s) {
  if (!s) return MK_ERR_INVALID_ARG;
  std::unique_lock<std::mutex> lk(s->mu);
  s->cv.wait(lk, [&] {
    if (s->status != MK_OK) return true;
    if (s->busy) return false;
    const bool admit = !s->pending.empty() && (int)s->rows.size() < s->max_batch;
    return s->budget == 0 || s->paused || (s->rows.empty() && !admit);
  });
  return s->status;
}

int32_t mk_server_poll(mk_server* s, int64_t* ids, int32_t* n_tokens, int32_t max) {
  if (!s || max < 0 || (max > 0 && (!ids || !n_tokens))) return -1;
  std::lock_guard<std::mutex> lk(s->mu);
  int32_t n = 0;
  for (auto& q : s->done) {
    if (n >= max) break;
    ids[n] = q.id;
    n_tokens[n] = (int32_t)q.out.size();
    ++n;
  }
  return n;
}

mk_status mk_server_take(mk_server* s, int64_t request_id, int32_t* tokens, int32_t cap, int32_t* n) {
  if (!s || !n || cap < 0 || (cap > 0 && !tokens)) return MK_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(s->mu);
  for (auto it = s->done.begin(); it != s->done.end(); ++it) {
    if (it->id != request_id) continue;
    if ((int32_t)it->out.size() > cap) { *n = (int32_t)it->out.size(); return MK_ERR_INVALID_ARG; }
    std::copy(it->out.begin(), it->out.end(), tokens);
    *n = (int32_t)it->out.size();
    s->done.erase(it);
    return MK_OK;
  }
  *n = 0;
  return MK_ERR_INVALID_ARG;
}

mk_status mk_server_stats(mk_server* s, mk_server_stats_t* out) {
  if (!s || !out) return MK_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(s->mu);
  out->steps = s->steps;
  out->tokens = s->tokens;
  out->rebuilds = s->rebuilds;
  out->active = (int32_t)s->rows.size();
  out->pending = (int32_t)s->pending.size();
  out->finished = (int32_t)s->done.size();
  out->paused = s->paused ? 1 : 0;
  out->busy_seconds = s->busy_s;
  out->prefill_tokens = s->prefill_tokens;
  return s->status;
}

mk_status mk_server_last_step(mk_server* s, mk_server_step* rec, const float** logits) {
  if (!s || !rec) return MK_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(s->mu);
  *rec = s->last;
  if (logits) *logits = s->logits_out ? s->logits_out : s->d_logits;
  return s->status;
}

mk_status mk_server_get_error(mk_server* s, char* buf, size_t n) {
  if (!s) return MK_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(s->mu);
  if (buf && n) {
    const size_t k = std::min(n - 1, s->msg.size());
    memcpy(buf, s->msg.data(), k);
    buf[k] = 0;
  }
  return s->status;
}

mk_status mk_server_destroy(mk_server* s) {
  if (!s) return MK_ERR_INVALID_ARG;
  {
    std::lock_guard<std::mutex> lk(s->mu);
    s->stop = true;
    s->cv.notify_all();
  }
  if (s->owner.joinable()) s->owner.join();
  const mk_status st = s->status;
  (void)hipStreamSynchronize(s->stream);
  (void)mk_set_step_outputs(s->e, nullptr, nullptr, nullptr, nullptr, nullptr);
  void* dp[] = {s->d_tokens, s->d_pos, s->d_lens, s->d_bt, s->d_argmax, s->d_logits};
  for (void* p : dp) if (p) (void)hipFree(p);
  (void)hipHostFree(s->h_in);
  (void)hipHostFree(s->h_argmax);
  (void)hipStreamDestroy(s->stream);
  delete s;
  return st;
}

}  // extern "C"
