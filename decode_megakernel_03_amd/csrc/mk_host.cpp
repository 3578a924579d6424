// Host side of libmk: model validation, workspace, the static task scheduler, a schedule validator,
// a CPU simulation of the persistent loop, and the C ABI declared in include/mk.h.
//
// Scheduling follows "mostly static" scheduling (P3 "Scheduling and Performance Benchmarks"): the
// host expands one decode step into tasks, groups them into topological levels (one parallel layer
// = four levels: QKV/router -> attention splits/expert slices -> attention merges -> output rows)
// and deals each level's tasks to the resident workers by a longest-first list schedule over an
// HBM-bytes cost model. At batch > 1 the expert slices are not dealt but drawn at run time from a
// per-layer work queue (dynamic work stealing): which experts a step needs is known only after
// the router.
// Tile counts are derived from the worker count rather than a fixed tile, so a level never ends
// with a partly filled wave of tiles (P1 "One persistent kernel for the whole decode step": wave
// quantization). Attention is split per KV group; each group's merges count on their own sub-counters
// of the layer's attention counter, so an output row may multiply a group's W_o columns as soon as
// that group's attention has landed (an ablation flag: measured slower than waiting for all groups).
// Weight loads are issued before dependency waits inside the kernel.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <numeric>
#include <random>
#include <string>
#include <vector>
#include <unordered_map>

#include "../../include/mk.h"
#include "mk_internal.h"
#include "mk_launch.h"

using namespace mk;

namespace {

struct Task {
  int32_t w[DESC_WORDS];
};

std::string fmt(const char* f, ...) {
  char buf[1024];
  va_list ap;
  va_start(ap, f);
  vsnprintf(buf, sizeof buf, f, ap);
  va_end(ap);
  return buf;
}

void put(char* buf, size_t n, const std::string& s) {
  if (!buf || n == 0) return;
  size_t k = std::min(n - 1, s.size());
  memcpy(buf, s.data(), k);
  buf[k] = 0;
}

struct Dims {
  int L, H, HQ, HKV, D, E, K, F, V, HPG, QKVR, AD, PART;
  int wb32;    // bytes per 32 matrix weights (64 bf16, 32 FP8, 17 MXFP4), for the schedule's cost model
  bool lm;
};

Dims dims_of(const mk_model_desc& d) {
  Dims m;
  m.L = d.n_layers; m.H = d.hidden; m.HQ = d.n_q_heads; m.HKV = d.n_kv_heads; m.D = d.head_dim;
  m.E = d.n_experts; m.K = d.top_k; m.F = d.expert_ffn; m.V = d.vocab;
  m.HPG = m.HQ / m.HKV; m.QKVR = (m.HQ + 2 * m.HKV) * m.D; m.AD = m.HQ * m.D;
  m.PART = m.HPG * (m.D + 2);
  m.wb32 = d.weight_format == MK_WEIGHTS_MXFP4 ? 17 : d.weight_format == MK_WEIGHTS_FP8 ? 32 : 64;
  m.lm = d.has_lm_head != 0;
  return m;
}

mk_status check_desc(const mk_model_desc* d, std::string* why) {
  if (!d) { *why = "desc is NULL"; return MK_ERR_INVALID_ARG; }
  if (d->abi_version != MK_ABI_VERSION) { *why = fmt("abi_version %d != %d", d->abi_version, MK_ABI_VERSION); return MK_ERR_INVALID_ARG; }
  if (d->n_layers < 1 || d->vocab < 1 || d->num_pages < 1 || d->max_pages_per_seq < 1) {
    *why = "n_layers, vocab, num_pages and max_pages_per_seq must be >= 1"; return MK_ERR_INVALID_ARG;
  }
  if (d->max_batch < 1 || d->max_batch > MK_MAX_BATCH) { *why = fmt("max_batch %d outside 1..%d", d->max_batch, MK_MAX_BATCH); return MK_ERR_INVALID_ARG; }
  if (d->page_size != PAGE) { *why = fmt("page_size %d unsupported (16)", d->page_size); return MK_ERR_UNSUPPORTED; }
  if (d->weight_format != MK_WEIGHTS_BF16 && d->weight_format != MK_WEIGHTS_FP8 && d->weight_format != MK_WEIGHTS_MXFP4) {
    *why = fmt("weight_format %d unknown", d->weight_format); return MK_ERR_INVALID_ARG;
  }
  if (shape_id(d->hidden, d->head_dim, d->n_q_heads, d->n_kv_heads, d->n_experts, d->top_k, d->expert_ffn,
               d->weight_format) < 0) {
    *why = "no compiled kernel for this (hidden, head_dim, heads, experts, top_k, expert_ffn)"; return MK_ERR_UNSUPPORTED;
  }
  if (!(d->rms_eps > 0.f) || !(d->rope_theta > 0.f)) { *why = "rms_eps and rope_theta must be > 0"; return MK_ERR_INVALID_ARG; }
  return MK_OK;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// counter indices of one schedule
struct Ctrs {
  int n = 0;
  int alloc(int k = 1) { int c = n; n += k; return c; }
};

}  // namespace

// ============================================================================== the plan

struct mk_plan {
  mk_model_desc desc;
  Dims m;
  int B = 0, n_workers = 0, split_keys = 0;
  std::vector<int> seq_lens;
  std::vector<Task> tasks;        // queue order: worker 0's tasks, worker 1's, ...
  std::vector<int32_t> qoff;      // n_workers + 1
  std::vector<int64_t> bytes;     // cost model, per task (queue order)
  int n_ctr = 0, done_ctr = 0, parts_per_layer = 0, n_attn = 0;
  std::vector<int> capacity;      // per sequence: largest seq_len the schedule can serve
  // most rows one sequence holds in a step (its consecutive positions), hence the most positions a
  // row advances per step; above 1 the QKV tasks publish the step's K/V (kernel instance 2)
  int rows_per_seq = 1;
};

namespace {

struct Proto {            // task before placement
  Task t;
  int64_t bytes;
  int prio;               // order inside a worker's level segment (lower first)
  int pin = -1;           // attention merge: placed on the worker of this split (b, g, s) key
};

void set(Task& t, int op, int layer, int level) {
  for (int i = 0; i < DESC_WORDS; ++i) t.w[i] = 0;
  t.w[D_OP] = op; t.w[D_LAYER] = layer; t.w[D_LEVEL] = level;
  t.w[D_W0] = t.w[D_W1] = t.w[D_SIG] = t.w[D_SIG2] = -1;
}

// Split [0, len) into n near-equal ranges.
std::vector<std::pair<int, int>> even(int len, int n) {
  std::vector<std::pair<int, int>> r;
  n = std::max(1, std::min(n, len));
  for (int i = 0; i < n; ++i) r.push_back({(int)((int64_t)len * i / n), (int)((int64_t)len * (i + 1) / n)});
  return r;
}

// Split [0, len) into consecutive ranges of `size` (the last one shorter).
std::vector<std::pair<int, int>> chunks(int len, int size) {
  std::vector<std::pair<int, int>> r;
  size = std::max(1, size);
  for (int a = 0; a < len; a += size) r.push_back({a, std::min(len, a + size)});
  return r;
}

mk_status build_plan(const mk_model_desc& desc, int B, const int32_t* seq_lens, int W, int split_req,
                     mk_plan* P, std::string* why, int flags = 0, int rows_per_seq = 1) {
  const Dims m = dims_of(desc);
  if (rows_per_seq < 1 || rows_per_seq > B) {
    *why = fmt("rows_per_seq = %d outside 1..batch (%d)", rows_per_seq, B);
    return MK_ERR_INVALID_ARG;
  }
  const bool kv_first = rows_per_seq > 1;
  P->desc = desc; P->m = m; P->B = B; P->n_workers = W; P->rows_per_seq = rows_per_seq;
  P->seq_lens.assign(seq_lens, seq_lens + B);
  const int SPLITMAX = split_max(), OUTR = out_max_rows();
  for (int b = 0; b < B; ++b) {
    if (seq_lens[b] < 1 || seq_lens[b] > desc.max_pages_per_seq * PAGE) {
      *why = fmt("seq_lens[%d] = %d outside 1..%d", b, seq_lens[b], desc.max_pages_per_seq * PAGE);
      return MK_ERR_INVALID_ARG;
    }
  }
  // Tile sizes. Every tile whose output another worker reads writes whole 64-byte sectors (16
  // floats) that no other tile writes: sectors written in parts by several workers made those
  // stores take several microseconds to complete under load, on the path of every consumer.
  const int slots = std::min(m.E, m.K * B);
  const int align = (m.F % 16 == 0) ? 16 : 1;
  auto splits_for = [&](int sp) {
    int n = 0;
    for (int b = 0; b < B; ++b) n += ((seq_lens[b] - 1) / sp + 1) * m.HKV;
    return n;
  };
  // attention split length: ~256 keys (128 KB of K+V) per task; long contexts use longer splits so
  // that a (sequence, KV group) never has more splits than one merge can combine (merge_max()), and
  // the last split keeps at least a quarter of SPLIT_MAX of room to grow before the schedule must
  // be rebuilt
  int maxlen = *std::max_element(seq_lens, seq_lens + B);
  // (with several sequences the splits alone fill the workers: two 256-key chunks per split halve
  // their count, measured +4 % at batch 8 over 256 keys; 384 and 768 keys were slower)
  int split = split_req > 0 ? split_req : (B > 1 ? 512 : 256);
  split = std::max(split, (int)ceil_div(ceil_div(maxlen, merge_max() - 8), 16) * 16);
  split = std::max(16, std::min(split, 3 * SPLITMAX / 4));
  split = (split + 15) / 16 * 16;
  // level 1 holds the attention splits and the expert slices: size the slices so that the level
  // has about one task per worker (tasks are latency-bound; a second task on a worker doubles its
  // part of the level), in whole sectors
  const int64_t gu_target = std::max<int64_t>(slots, W - splits_for(split));
  int nf = (int)ceil_div(m.F, std::max<int64_t>(1, gu_target / slots));
  nf = std::max(4, std::min(32, nf));   // at most 256 KB of gate + up per task (balance at large batches)
  // with several sequences the slices are queue items: 16 rows, which the kernel takes three at a
  // time (two for MXFP4 rows) when the step's union is large (see the expert queue in the kernel)
  if (B > 1 && !(flags & MK_FLAG_STATIC_EXPERTS)) nf = 16;
  if (align > 1) nf = std::max(align, (nf + align / 2) / align * align);
  const int slices = (int)ceil_div(m.F, nf);
  // with several sequences (the expert queue), the longest splits that keep enough of them for
  // level 0 to spread over every worker (see lvl0_budget below): fewer attention tasks leave more
  // workers free to start on the experts right after the router. Measured on MI355X at batch 8,
  // 8K context: 512 keys (512 splits) 1055 tok/s, 688-736 keys (384 splits) 1077-1090, 752 keys
  // (352 splits: level 0 squeezed onto the workers left over) 1029.
  const int router_tiles_ = std::max(1, std::min(8, m.E / 16));
  if (split_req <= 0 && B > 1 && !(flags & MK_FLAG_STATIC_EXPERTS)) {
    const int keep = W - W / 4 - router_tiles_ - 3 * m.HKV;    // splits needed to keep level 0 spread
    for (int sp = split + 16; sp <= 3 * SPLITMAX / 4 && splits_for(sp) > keep; sp += 16) split = sp;
  }
  // if slices and splits then exceed one task per worker, lengthen the splits (up to twice the
  // default) until they fit
  if (split_req <= 0)
    for (int sp = split; sp <= std::min(2 * split, 3 * SPLITMAX / 4); sp += 16)
      if (splits_for(sp) + slots * slices <= W) { split = sp; break; }
  P->split_keys = split;

  Ctrs C;
  const int L = m.L;
  std::vector<int> c_x(L + 1, -1), c_rarr(L), c_route(L), c_h(L), c_att(L);
  std::vector<std::vector<int>> c_qkv(L, std::vector<int>(m.HKV));
  std::vector<std::vector<int>> c_aarr(L, std::vector<int>(B * m.HKV));
  // expert slices drawn from a per-layer queue (dynamic work stealing) unless static slices are
  // asked for; the queue is a counter of its own (zeroed with the others at the end of a step).
  // At batch 1 the union is always top_k experts, so the work is known before the step and the
  // static deal is kept (measured: the queue only moves items between equally loaded workers).
  const bool steal = B > 1 && !(flags & MK_FLAG_STATIC_EXPERTS);
  // down items per union slot (row blocks of W_down[e], DOWN_ROWS rows each) in queue mode
  const int down_items = steal ? (int)ceil_div(m.H, down_rows()) : 0;
  // O-projection row blocks of OPROJ_ROWS rows, queued between the gate/up and the down items (bf16
  // and MXFP4 matrices: the FP8 kernel instances are compiled without them); the output rows then
  // only add up
  constexpr int OPROJ_ROWS = 16;
  // (each row block once per group of 4 tokens: the kernel's items stage 4 tokens' attention)
  const int oproj_items = steal && desc.weight_format != MK_WEIGHTS_FP8
                        ? (int)ceil_div(m.H, OPROJ_ROWS) * (int)ceil_div(B, 4) : 0;
  std::vector<int> c_queue(L, -1);
  for (int l = 0; l < L; ++l) {
    for (int g = 0; g < m.HKV; ++g) c_qkv[l][g] = C.alloc();
    // the attention counter: the merges of KV group g add to its sub-counters g * (CTR_SUB / HKV) ..,
    // so an output row can also see each group's attention land on its own (P1 "One persistent kernel
    // for the whole decode step")
    c_rarr[l] = C.alloc(); c_route[l] = C.alloc(); c_h[l] = C.alloc(); c_att[l] = C.alloc();
    if (steal) c_queue[l] = C.alloc();
    for (int i = 0; i < B * m.HKV; ++i) c_aarr[l][i] = C.alloc();
    c_x[l + 1] = C.alloc();
  }
  P->done_ctr = C.alloc();
  P->n_ctr = C.n;

  // tile sizes from the worker count
  const int router_tiles = std::max(1, std::min(8, m.E / 16));
  // attention splits per sequence: [k0, k0 + split) ... last split open-ended from k0_last
  std::vector<int> nsplit(B), pbase_b(B);
  int parts = 0;
  P->capacity.resize(B);
  for (int b = 0; b < B; ++b) {
    const int pos = seq_lens[b] - 1;
    const int k0_last = pos / split * split;
    nsplit[b] = k0_last / split + 1;
    pbase_b[b] = parts;
    parts += nsplit[b] * m.HKV;
    P->capacity[b] = std::min(k0_last + SPLITMAX, desc.max_pages_per_seq * PAGE);
  }
  P->parts_per_layer = parts;
  // level 0 holds QKV tiles and router tiles. Size the QKV tiles so that level 0 leaves a worker
  // free for every attention split: those workers reach their split at the start of the layer and
  // its keys stream in while level 0 runs (old keys do not depend on the step's activations).
  // When the splits alone fill the workers (large batches), no worker can be kept free for them
  // and level 0 spreads over every worker instead.
  const int lvl0_budget = parts + router_tiles + 3 * m.HKV + W / 4 <= W ? W - parts - router_tiles - 3 * m.HKV
                                                                       : W - router_tiles;
  int qkv_tile = std::max(4, std::min(64, (int)ceil_div(m.QKVR, lvl0_budget)));
  if (m.D % 16 == 0) qkv_tile = std::min(m.D, (qkv_tile + 15) / 16 * 16);   // whole sectors

  // levels per layer: QKV + router | attention splits + expert slices | attention merges | output rows
  constexpr int LPL = 4;
  const int nslice = std::max(1, m.HPG * m.D / 256);       // merge tasks per (sequence, KV group)
  // output rows: OUT_ROWS per task, except that the workers of the attention merges, which reach
  // their OUT task only after the merge, get none when the others can take every row in tasks of
  // at most OUTR rows
  constexpr int OUT_ROWS = 4;
  const int n_merge = B * m.HKV * nslice;
  int n_out_l = (int)ceil_div(m.H, std::min(OUT_ROWS, OUTR));
  if (W - n_merge >= (int)ceil_div(m.H, OUTR)) n_out_l = std::min(n_out_l, W - n_merge);
  auto split_key = [&](int l, int b, int g, int s) { return ((l * B + b) * m.HKV + g) * 65536 + s; };
  std::vector<std::vector<Proto>> levels(LPL * L + 1);
  int n_out_layer = 0;                      // output-row tasks per layer when they are not n_out_l
  int n_attn = 0;
  for (int l = 0; l < L; ++l) {
    const int lv0 = LPL * l, lv1 = LPL * l + 1, lvm = LPL * l + 2, lv2 = LPL * l + 3;
    // level 0: QKV rows (per KV group: q heads, k, v) and router tiles
    std::vector<int> qkv_count(m.HKV, 0);
    for (int g = 0; g < m.HKV; ++g) {
      const int regions[3][2] = {{g * m.HPG * m.D, m.HPG * m.D}, {m.HQ * m.D + g * m.D, m.D}, {(m.HQ + m.HKV) * m.D + g * m.D, m.D}};
      for (int ri = 0; ri < 3; ++ri) {
        const auto& rg = regions[ri];
        // when the QKV tasks publish the step's keys, a K tile is one whole head (RoPE pairs dims
        // d and d + D/2) and V tiles hold whole 16-byte groups of 8 dims
        const int tile = !kv_first ? qkv_tile : ri == 1 ? m.D : std::max(8, qkv_tile / 8 * 8);
        for (auto [a, e] : chunks(rg[1], tile)) {
          Proto pr;
          set(pr.t, OP_QKV, l, lv0);
          pr.t.w[D_A0] = rg[0] + a; pr.t.w[D_A1] = e - a;
          pr.t.w[D_W0] = c_x[l]; pr.t.w[D_T0] = -1;   // target filled below
          pr.t.w[D_SIG] = c_qkv[l][g];
          pr.bytes = (int64_t)(e - a) * m.H * m.wb32 / 32;
          pr.prio = 1;
          levels[lv0].push_back(pr);
          qkv_count[g]++;
        }
      }
    }
    for (auto [a, e] : even(m.E, router_tiles)) {
      Proto pr;
      set(pr.t, OP_ROUTER, l, lv0);
      pr.t.w[D_A0] = a; pr.t.w[D_A1] = e - a; pr.t.w[D_A2] = router_tiles;
      pr.t.w[D_W0] = c_x[l]; pr.t.w[D_T0] = -1;   // target filled below
      pr.t.w[D_SIG] = c_rarr[l]; pr.t.w[D_SIG2] = c_route[l];
      pr.bytes = (int64_t)(e - a) * m.H * m.wb32 / 32;
      pr.prio = 0;
      levels[lv0].push_back(pr);
    }
    // level 1: attention splits (each writes its partial and signals its group's arrival
    // counter), expert slices
    for (int b = 0; b < B; ++b)
      for (int g = 0; g < m.HKV; ++g)
        for (int s = 0; s < nsplit[b]; ++s) {
          Proto pr;
          set(pr.t, OP_ATTN, l, lv1);
          const int k0 = s * split;
          const bool last = s == nsplit[b] - 1;
          pr.t.w[D_A0] = b; pr.t.w[D_A1] = g; pr.t.w[D_A2] = k0; pr.t.w[D_A3] = last ? -1 : k0 + split;
          pr.t.w[D_A4] = pbase_b[b] + g * nsplit[b];
          pr.t.w[D_A5] = s | (nsplit[b] << 16);
          pr.t.w[D_W0] = c_qkv[l][g]; pr.t.w[D_T0] = qkv_count[g];
          pr.t.w[D_SIG] = c_aarr[l][b * m.HKV + g];
          const int keys = last ? seq_lens[b] - k0 : split;
          pr.bytes = (int64_t)keys * m.D * 2 * 2;
          pr.prio = 0;
          pr.pin = -2 - split_key(l, b, g, s);     // records its worker (see placement)
          levels[lv1].push_back(pr);
          n_attn++;
        }
    int n_gu = 0;
    if (steal) {
      // one task per worker at most: each draws (slot, slice) items until the queue is empty, so
      // the routing-dependent expert work goes to whichever workers are free first
      // the down projection of every union expert joins the queue as row blocks (after every gate/up
      // item), so that W_down is read once per expert and streams while other slots' gate/up items
      // are still running; the output rows then only add the experts' results
      const int n_items = slots * (slices + down_items) + oproj_items;
      const int tickets = std::min(n_items, W);
      const int nq = std::min(CTR_SUB, tickets);
      // the tickets follow the attention merges in each worker's queue (same level, after them):
      // a merge then runs as soon as its group's splits are in, instead of after that worker has
      // drained the queue (measured on MI355X: +0.6 % at batch 8)
      for (int t = 0; t < tickets; ++t) {
        Proto pr;
        set(pr.t, OP_GATEUP, l, lvm);
        pr.t.w[D_A0] = t % nq; pr.t.w[D_A1] = nq; pr.t.w[D_A2] = slices; pr.t.w[D_A3] = c_queue[l];
        pr.t.w[D_A4] = nf; pr.t.w[D_A5] = down_items | (oproj_items << 16);
        pr.t.w[D_W0] = c_x[l]; pr.t.w[D_T0] = -1;        // x_l complete (target filled below)
        pr.t.w[D_W1] = c_rarr[l]; pr.t.w[D_T1] = router_tiles;   // every router logit written
        pr.t.w[D_SIG] = c_h[l];
        pr.bytes = ((int64_t)slots * slices * 2 * nf * m.H * m.wb32 / 32 + (int64_t)slots * m.H * m.F * m.wb32 / 32) / tickets;
        pr.prio = 1;
        levels[lvm].push_back(pr);
        n_gu++;
      }
    } else {
      for (int u = 0; u < slots; ++u)
        for (int j = 0; j < slices; ++j) {
          Proto pr;
          set(pr.t, OP_GATEUP, l, lv1);
          const int f0 = j * nf, f1 = std::min(m.F, f0 + nf);
          pr.t.w[D_A0] = u; pr.t.w[D_A1] = f0; pr.t.w[D_A2] = f1 - f0; pr.t.w[D_A3] = -1;
          pr.t.w[D_W0] = c_x[l]; pr.t.w[D_T0] = -1;        // x_l complete (target filled below)
          pr.t.w[D_W1] = c_rarr[l]; pr.t.w[D_T1] = router_tiles;   // every router logit written
          pr.t.w[D_SIG] = c_h[l];
          pr.bytes = (int64_t)2 * (f1 - f0) * m.H * m.wb32 / 32;
          pr.prio = 1;
          levels[lv1].push_back(pr);
          n_gu++;
        }
    }
    // level 2: attention merges, nslice per (sequence, KV group), each on the worker of one of the
    // group's splits (that worker is done with the step's heavy streams by then)
    for (int b = 0; b < B; ++b)
      for (int g = 0; g < m.HKV; ++g)
        for (int q = 0; q < nslice; ++q) {
          Proto pr;
          set(pr.t, OP_MERGE, l, lvm);
          pr.t.w[D_A0] = b; pr.t.w[D_A1] = g; pr.t.w[D_A2] = q; pr.t.w[D_A3] = nslice;
          pr.t.w[D_A4] = pbase_b[b] + g * nsplit[b]; pr.t.w[D_A5] = nsplit[b];
          pr.t.w[D_W0] = c_aarr[l][b * m.HKV + g]; pr.t.w[D_T0] = nsplit[b];
          pr.t.w[D_SIG] = c_att[l];
          pr.bytes = (int64_t)nsplit[b] * m.HPG * (m.D + 2) * 4 / nslice;
          pr.prio = 0;
          pr.pin = split_key(l, b, g, (int)((int64_t)q * nsplit[b] / nslice));
          levels[lvm].push_back(pr);
        }
    // level 3: output rows (O-proj + expert down-proj + residual); with queued O-projection items,
    // x_l+1 = (x_l + o) + MoE term in blocks of up to 32 rows (one thread per row and token)
    int n_out = 0;
    if (oproj_items > 0)
      for (auto [a, e] : chunks(m.H, std::max(1, std::min(32, NT / B)))) {
        Proto pr;
        set(pr.t, OP_OUT, l, lv2);
        pr.t.w[D_A0] = a; pr.t.w[D_A1] = e - a;
        pr.t.w[D_A2] = c_att[l]; pr.t.w[D_A3] = B * m.HKV * nslice;   // (every merge: already in)
        pr.t.w[D_A4] = 4 | 1;
        pr.t.w[D_W0] = c_route[l]; pr.t.w[D_T0] = 1;
        pr.t.w[D_W1] = c_h[l]; pr.t.w[D_T1] = n_gu;
        pr.t.w[D_SIG] = c_x[l + 1];
        pr.bytes = (int64_t)(e - a) * B * (m.K + 2) * 4;
        pr.prio = 0;
        levels[lv2].push_back(pr);
        n_out++;
      }
    if (oproj_items > 0) n_out_layer = n_out;
    if (oproj_items == 0)
    for (auto [a, e] : even(m.H, n_out_l)) {
      Proto pr;
      set(pr.t, OP_OUT, l, lv2);
      pr.t.w[D_A0] = a; pr.t.w[D_A1] = e - a;
      pr.t.w[D_A2] = c_att[l]; pr.t.w[D_A3] = B * m.HKV * nslice;   // every merge of every KV group
      pr.t.w[D_A4] = down_items > 0 ? 1 : 0;
      pr.t.w[D_W0] = c_route[l]; pr.t.w[D_T0] = 1;
      pr.t.w[D_W1] = c_h[l]; pr.t.w[D_T1] = n_gu;
      pr.t.w[D_SIG] = c_x[l + 1];
      pr.bytes = (int64_t)(e - a) * (m.AD + (down_items > 0 ? 0 : (int64_t)slots * m.F)) * m.wb32 / 32;
      pr.prio = 0;
      levels[lv2].push_back(pr);
      n_out++;
    }
    // targets of the waits on x_l+1 (next layer's level 0, or lm_head)
    for (int lv = 0; lv < (int)levels.size(); ++lv) (void)lv;
    P->n_attn = n_attn;
    // fill T0 of the next layer's x waits once its producers are known
    if (l + 1 < L) {
      // placeholder: set after the loop (producer counts are identical per layer)
    }
    (void)n_out;
  }
  const int n_out_per_layer = n_out_layer > 0 ? n_out_layer : n_out_l;
  for (auto& lvl : levels)
    for (auto& pr : lvl)
      if ((pr.t.w[D_OP] == OP_QKV || pr.t.w[D_OP] == OP_ROUTER || pr.t.w[D_OP] == OP_GATEUP) && pr.t.w[D_W0] >= 0 &&
          pr.t.w[D_T0] < 0)
        pr.t.w[D_T0] = n_out_per_layer;
  if (m.lm) {
    for (auto [a, e] : even(m.V, W)) {
      Proto pr;
      set(pr.t, OP_LMHEAD, L, LPL * L);
      pr.t.w[D_A0] = a; pr.t.w[D_A1] = e - a;
      pr.t.w[D_W0] = c_x[L]; pr.t.w[D_T0] = n_out_per_layer;
      pr.bytes = (int64_t)(e - a) * m.H * m.wb32 / 32;
      pr.prio = 0;
      levels[LPL * L].push_back(pr);
    }
  }

  // Every task pays a fixed latency (dependency poll, activation round trip, drain) worth about
  // TASK_FIXED bytes of streaming; attention also pays for its arithmetic (8 query heads per key).
  // The term is large on purpose: a second task on a worker in one level costs its hops in full,
  // so the placement balances task counts first and bytes second (measured on MI355X: 48, 96, 192,
  // 288, 384 KB -> 561, 563, 570, 574, 573 tok/s at batch 1; 288 KB also best at batch 8).
  const int64_t TASK_FIXED = 288 * 1024;
  for (auto& lvl : levels)
    for (auto& pr : lvl) pr.bytes = pr.bytes * (pr.t.w[D_OP] == OP_ATTN ? 2 : 1) + TASK_FIXED;
  // placement: per level, longest task first onto the worker with the least load in that level;
  // ties go to the worker with the least load in the previous level (so attention splits land on
  // workers idle in level 0 and prefetch their keys early), then least total load, then index.
  // Each worker's queue is level-ordered, and inside a level its tasks run in priority order
  // (router before QKV, attention before expert slices).
  // each worker's queue as (level, index in level) references; the descriptors are copied once, at the end
  struct Ref { int32_t lv, idx; };
  std::vector<std::vector<Ref>> queues(W);
  {
    size_t ntask = 0;
    for (auto& lvl : levels) ntask += lvl.size();
    for (auto& q : queues) q.reserve(ntask / W + 16);
  }
  std::unordered_map<int, int> split_worker;                    // attention split key -> worker
  std::vector<int64_t> total(W, 0), prev(W, 0);
  std::vector<char> merge_w(W, 0);                              // workers with a merge this layer
  constexpr int64_t AVOID = (int64_t)1 << 50;
  std::vector<int64_t> lload(W, 0);
  // the workers in a binary min-heap on (level load, previous level load, total load, index): the
  // worker a task goes to is the heap's top, exactly the first minimum of a scan in index order
  std::vector<int> heap(W), at(W);
  auto less = [&](int a, int b) {
    return lload[a] != lload[b] ? lload[a] < lload[b] : prev[a] != prev[b] ? prev[a] < prev[b]
         : total[a] != total[b] ? total[a] < total[b] : a < b;
  };
  auto put = [&](int i, int w) { heap[i] = w; at[w] = i; };
  auto sift_down = [&](int i) {
    const int w = heap[i];
    for (;;) {
      int c = 2 * i + 1;
      if (c >= W) break;
      if (c + 1 < W && less(heap[c + 1], heap[c])) ++c;
      if (!less(heap[c], w)) break;
      put(i, heap[c]);
      i = c;
    }
    put(i, w);
  };
  for (int lv = 0; lv < (int)levels.size(); ++lv) {
    auto& lvl = levels[lv];
    std::vector<int> order(lvl.size());
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return lvl[a].bytes > lvl[b].bytes; });
    std::fill(lload.begin(), lload.end(), 0);
    // output rows avoid the merge workers only when the others can take one output task each
    const bool out_level = lv < LPL * L && lv % LPL == LPL - 1 && W - n_merge >= n_out_l;
    if (out_level)
      for (int w = 0; w < W; ++w) lload[w] = merge_w[w] ? AVOID : 0;
    // merges first go to their fixed workers (placement of the others only sees the sums), then
    // the heap is built over the level's starting loads
    for (int idx : order) {
      if (lvl[idx].pin < 0) continue;          // attention merge: on the worker of its split
      const int w = split_worker.at(lvl[idx].pin);
      merge_w[w] = 1;
      lload[w] += lvl[idx].bytes;
      total[w] += lvl[idx].bytes;
      queues[w].push_back({lv, idx});
    }
    for (int w = 0; w < W; ++w) put(w, w);
    for (int i = W / 2 - 1; i >= 0; --i) sift_down(i);
    for (int idx : order) {
      if (lvl[idx].pin >= 0) continue;
      const int best = heap[0];
      lload[best] += lvl[idx].bytes;           // only the top's key grows: restore the heap below it
      total[best] += lvl[idx].bytes;
      sift_down(0);
      queues[best].push_back({lv, idx});
      if (lvl[idx].pin <= -2) split_worker[-2 - lvl[idx].pin] = best;
    }
    if (out_level) {
      for (int w = 0; w < W; ++w) if (merge_w[w]) lload[w] -= AVOID;
      std::fill(merge_w.begin(), merge_w.end(), 0);
    }
    prev = lload;
  }
  P->tasks.clear(); P->bytes.clear(); P->qoff.assign(W + 1, 0);
  {
    size_t ntask = 0;
    for (auto& q : queues) ntask += q.size();
    P->tasks.reserve(ntask);
    P->bytes.reserve(ntask);
  }
  for (int w = 0; w < W; ++w) {
    auto& q = queues[w];
    std::stable_sort(q.begin(), q.end(), [&](const Ref& a, const Ref& b) {
      return a.lv != b.lv ? a.lv < b.lv : levels[a.lv][a.idx].prio < levels[b.lv][b.idx].prio;
    });
    P->qoff[w] = (int32_t)P->tasks.size();
    for (const Ref& r : q) {
      const Proto& pr = levels[r.lv][r.idx];
      P->tasks.push_back(pr.t);
      P->tasks.back().w[D_ID] = (int32_t)P->tasks.size() - 1;
      P->bytes.push_back(pr.bytes);
    }
  }
  P->qoff[W] = (int32_t)P->tasks.size();
  return MK_OK;
}

// Every (counter, target) a task waits for: W0/T0, W1/T1, and for an output-row task the attention
// counter A2 (every merge of the layer, A3).
struct Waits {
  int n = 0;
  std::array<std::array<int, 2>, 3> w;
  const std::array<int, 2>* begin() const { return w.data(); }
  const std::array<int, 2>* end() const { return w.data() + n; }
};
Waits task_waits(const Task& t, int hkv) {
  Waits w;
  if (t.w[D_W0] >= 0) w.w[w.n++] = {t.w[D_W0], t.w[D_T0]};
  if (t.w[D_W1] >= 0) w.w[w.n++] = {t.w[D_W1], t.w[D_T1]};
  if (t.w[D_OP] == OP_OUT) w.w[w.n++] = {t.w[D_A2], t.w[D_A3]};
  return w;
}

// ---- validation --------------------------------------------------------------------------

mk_status validate_plan(const mk_plan& P, std::string* why) {
  const Dims& m = P.m;
  const int nt = (int)P.tasks.size();
  std::vector<int> sig(P.n_ctr, 0);
  std::map<int, std::vector<int>> sig2_groups;      // SIG2 counter -> SIG counters feeding it
  std::vector<int> prod_level(P.n_ctr, -1);
  for (auto& t : P.tasks) {
    const int s = t.w[D_SIG], s2 = t.w[D_SIG2], lv = t.w[D_LEVEL];
    if (s >= P.n_ctr || s2 >= P.n_ctr || t.w[D_W0] >= P.n_ctr || t.w[D_W1] >= P.n_ctr) { *why = fmt("task %d: counter index out of range", t.w[D_ID]); return MK_ERR_INVALID_ARG; }
    if (s >= 0) { sig[s]++; prod_level[s] = std::max(prod_level[s], lv); }
    if (s2 >= 0) {
      if (s < 0) {
        sig[s2]++;                          // signalled once by this task
      } else {                              // signalled once by the last arriver of counter s
        auto& v = sig2_groups[s2];
        if (std::find(v.begin(), v.end(), s) == v.end()) v.push_back(s);
      }
      prod_level[s2] = std::max(prod_level[s2], lv);
    }
    if (s == P.done_ctr || s2 == P.done_ctr) { *why = "a task signals the end-of-step counter"; return MK_ERR_INVALID_ARG; }
  }
  for (auto& [c, v] : sig2_groups) sig[c] += (int)v.size();
  for (auto& t : P.tasks) {
    const auto waits = task_waits(t, m.HKV);
    for (auto& wt : waits) {
      if (wt[0] < 0) continue;
      if (wt[0] >= P.n_ctr) { *why = fmt("task %d waits on counter %d of %d", t.w[D_ID], wt[0], P.n_ctr); return MK_ERR_INVALID_ARG; }
      if (wt[1] != sig[wt[0]]) { *why = fmt("task %d (op %d) waits for counter %d >= %d but %d signals exist", t.w[D_ID], t.w[D_OP], wt[0], wt[1], sig[wt[0]]); return MK_ERR_INVALID_ARG; }
      if (prod_level[wt[0]] >= t.w[D_LEVEL]) { *why = fmt("task %d (level %d) depends on counter %d produced at level %d", t.w[D_ID], t.w[D_LEVEL], wt[0], prod_level[wt[0]]); return MK_ERR_INVALID_ARG; }
    }
    if (t.w[D_OP] == OP_ROUTER && t.w[D_A2] != sig[t.w[D_SIG]]) { *why = fmt("router task %d expects %d tiles, %d exist", t.w[D_ID], t.w[D_A2], sig[t.w[D_SIG]]); return MK_ERR_INVALID_ARG; }
    if (t.w[D_OP] == OP_MERGE && t.w[D_A5] != sig[t.w[D_W0]]) { *why = fmt("merge task %d expects %d splits, %d exist", t.w[D_ID], t.w[D_A5], sig[t.w[D_W0]]); return MK_ERR_INVALID_ARG; }
  }
  for (int w = 0; w < P.n_workers; ++w)
    for (int i = P.qoff[w] + 1; i < P.qoff[w + 1]; ++i)
      if (P.tasks[i].w[D_LEVEL] < P.tasks[i - 1].w[D_LEVEL]) { *why = fmt("worker %d queue is not level-ordered at task %d", w, i); return MK_ERR_INVALID_ARG; }
  // coverage: each output written exactly once (tasks visited per layer; counters that any task
  // waits on or signals marked once)
  std::vector<std::vector<const Task*>> by_layer(m.L);
  std::vector<char> ctr_used(P.n_ctr, 0);
  for (auto& t : P.tasks) {
    if (t.w[D_LAYER] >= 0 && t.w[D_LAYER] < m.L) by_layer[t.w[D_LAYER]].push_back(&t);
    if (t.w[D_SIG] >= 0) ctr_used[t.w[D_SIG]] = 1;
    if (t.w[D_SIG2] >= 0) ctr_used[t.w[D_SIG2]] = 1;
    for (auto& wt : task_waits(t, m.HKV)) if (wt[0] >= 0) ctr_used[wt[0]] = 1;
  }
  if (P.rows_per_seq > 1)
    for (auto& t : P.tasks) {
      if (t.w[D_OP] != OP_QKV || t.w[D_A0] < m.HQ * m.D) continue;
      const bool is_k = t.w[D_A0] < (m.HQ + m.HKV) * m.D;
      const int dlo = (t.w[D_A0] - (is_k ? m.HQ : m.HQ + m.HKV) * m.D) % m.D, n = t.w[D_A1];
      if (is_k ? (dlo != 0 || n != m.D) : (dlo % 8 != 0 || n % 8 != 0 || dlo + n > m.D)) {
        *why = fmt("task %d: a %s tile [%d, +%d) the QKV task cannot publish", t.w[D_ID], is_k ? "K" : "V", t.w[D_A0], n);
        return MK_ERR_INVALID_ARG;
      }
    }
  for (int l = 0; l < m.L; ++l) {
    std::vector<int> qkv(m.QKVR, 0), out(m.H, 0), rt(m.E, 0);
    std::map<int, std::vector<int>> gu;
    std::vector<std::vector<std::pair<int, int>>> att(P.B * m.HKV), mrg(P.B * m.HKV);
    std::vector<const Task*> queue_tasks;
    for (const Task* tp : by_layer[l]) {
      const Task& t = *tp;
      switch (t.w[D_OP]) {
        case OP_QKV: for (int r = t.w[D_A0]; r < t.w[D_A0] + t.w[D_A1]; ++r) qkv[r]++; break;
        case OP_ROUTER: for (int r = t.w[D_A0]; r < t.w[D_A0] + t.w[D_A1]; ++r) rt[r]++; break;
        case OP_OUT:
          if ((t.w[D_A4] & ~5) || ((t.w[D_A4] & 4) && (!(t.w[D_A4] & 1) || P.B * t.w[D_A1] > NT))) {
            *why = fmt("output task %d: mode %d with %d rows", t.w[D_ID], t.w[D_A4], t.w[D_A1]); return MK_ERR_INVALID_ARG;
          }
          for (int r = t.w[D_A0]; r < t.w[D_A0] + t.w[D_A1]; ++r) out[r]++;
          break;
        case OP_GATEUP: {
          if (t.w[D_A3] >= 0) { queue_tasks.push_back(&t); break; }
          auto& v = gu[t.w[D_A0]];
          v.resize(m.F, 0);
          for (int f = t.w[D_A1]; f < t.w[D_A1] + t.w[D_A2]; ++f) v[f]++;
          break;
        }
        case OP_ATTN:
        case OP_MERGE: {
          const int b = t.w[D_A0], g = t.w[D_A1];
          if (b < 0 || b >= P.B || g < 0 || g >= m.HKV) { *why = fmt("task %d: sequence %d group %d out of range", t.w[D_ID], b, g); return MK_ERR_INVALID_ARG; }
          (t.w[D_OP] == OP_ATTN ? att : mrg)[b * m.HKV + g].push_back({t.w[D_A2], t.w[D_A3]});
          break;
        }
      }
    }
    for (int r = 0; r < m.QKVR; ++r) if (qkv[r] != 1) { *why = fmt("layer %d qkv row %d written %d times", l, r, qkv[r]); return MK_ERR_INVALID_ARG; }
    for (int r = 0; r < m.E; ++r) if (rt[r] != 1) { *why = fmt("layer %d router row %d written %d times", l, r, rt[r]); return MK_ERR_INVALID_ARG; }
    for (int r = 0; r < m.H; ++r) if (out[r] != 1) { *why = fmt("layer %d output row %d written %d times", l, r, out[r]); return MK_ERR_INVALID_ARG; }
    if (!queue_tasks.empty()) {
      // queue mode: one queue counter per layer that no task waits on or signals; its items cover
      // every FFN row of every union slot once; every sub-queue has a task that drains it
      if (!gu.empty()) { *why = fmt("layer %d mixes static and queued expert slices", l); return MK_ERR_INVALID_ARG; }
      const Task& t0 = *queue_tasks[0];
      const int qc = t0.w[D_A3], nq = t0.w[D_A1], slices = t0.w[D_A2], nfs = t0.w[D_A4], qd = t0.w[D_A5] & 0xffff;
      const int n_oi = t0.w[D_A5] >> 16;
      // O-projection items: bf16 and MXFP4 matrices only; they wait on counter qc - 1, which must be the
      // attention counter the layer's output rows name; every output row then adds o
      if (n_oi < 0 || n_oi > m.H * (int)ceil_div(P.B, 4) || n_oi % (int)ceil_div(P.B, 4) != 0 ||
          (n_oi > 0 && P.desc.weight_format == MK_WEIGHTS_FP8)) {
        *why = fmt("layer %d: %d O-projection items", l, n_oi); return MK_ERR_INVALID_ARG;
      }
      for (const Task* tp : by_layer[l])
        if (tp->w[D_OP] == OP_OUT && (((tp->w[D_A4] & 4) != 0) != (n_oi > 0) ||
            (n_oi > 0 && (tp->w[D_A2] != qc - 1 || tp->w[D_A3] != P.B * m.HKV * std::max(1, m.HPG * m.D / 256))))) {
          // (the kernel's O-projection items wait for B * HKV * max(1, HPG * D / 256) merges on qc - 1)
          *why = fmt("layer %d: output task %d and the O-projection items disagree", l, tp->w[D_ID]);
          return MK_ERR_INVALID_ARG;
        }
      // down items: none, or row blocks that cover every W_down row once
      if (qd < 0 || (qd > 0 && (qd * down_rows() < m.H || (qd - 1) * down_rows() >= m.H))) {
        *why = fmt("layer %d: %d down items of %d rows for %d rows", l, qd, down_rows(), m.H);
        return MK_ERR_INVALID_ARG;
      }
      for (const Task* tp : by_layer[l])
        if (tp->w[D_OP] == OP_OUT && (tp->w[D_A4] & 1) != (qd > 0 ? 1 : 0)) {
          *why = fmt("layer %d: output task %d and the expert queue disagree on the down items", l, tp->w[D_ID]);
          return MK_ERR_INVALID_ARG;
        }
      if (qc >= P.n_ctr || nq < 1 || nq > CTR_SUB || slices < 1 || nfs < 1 || slices * nfs < m.F || (slices - 1) * nfs >= m.F) {
        *why = fmt("layer %d: bad expert queue (counter %d, %d sub-queues, %d slices of %d rows)", l, qc, nq, slices, nfs);
        return MK_ERR_INVALID_ARG;
      }
      std::vector<int> drained(nq, 0);
      for (const Task* t : queue_tasks) {
        if (t->w[D_A3] != qc || t->w[D_A1] != nq || t->w[D_A2] != slices || t->w[D_A4] != nfs || t->w[D_A5] != t0.w[D_A5] ||
            t->w[D_A0] < 0 || t->w[D_A0] >= nq) {
          *why = fmt("layer %d: expert task %d disagrees on the queue", l, t->w[D_ID]);
          return MK_ERR_INVALID_ARG;
        }
        drained[t->w[D_A0]]++;
      }
      for (int q = 0; q < nq; ++q) if (!drained[q]) { *why = fmt("layer %d: expert sub-queue %d has no task", l, q); return MK_ERR_INVALID_ARG; }
      if (qc >= 0 && ctr_used[qc]) { *why = fmt("a task waits on or signals the expert queue counter %d", qc); return MK_ERR_INVALID_ARG; }
    } else if ((int)gu.size() != std::min(m.E, m.K * P.B)) { *why = fmt("layer %d: %zu expert slots", l, gu.size()); return MK_ERR_INVALID_ARG; }
    if (queue_tasks.empty())
      for (const Task* tp : by_layer[l])
        if (tp->w[D_OP] == OP_OUT && tp->w[D_A4] != 0) {   // (no queue: no queued items to add)
          *why = fmt("layer %d: output task %d expects queued down items, the layer has none", l, tp->w[D_ID]);
          return MK_ERR_INVALID_ARG;
        }
    for (auto& [u, v] : gu) for (int f = 0; f < m.F; ++f) if (v[f] != 1) { *why = fmt("layer %d slot %d ffn row %d written %d times", l, u, f, v[f]); return MK_ERR_INVALID_ARG; }
    for (int b = 0; b < P.B; ++b)
      for (int g = 0; g < m.HKV; ++g) {
        auto& v = att[b * m.HKV + g];
        std::sort(v.begin(), v.end());
        int k = 0;
        for (size_t i = 0; i < v.size(); ++i) {
          if (v[i].first != k) { *why = fmt("layer %d seq %d group %d: key ranges leave a gap at %d", l, b, g, k); return MK_ERR_INVALID_ARG; }
          const bool last = i + 1 == v.size();
          if (last != (v[i].second < 0)) { *why = fmt("layer %d seq %d group %d: only the last split may be open", l, b, g); return MK_ERR_INVALID_ARG; }
          k = v[i].second;
        }
        if (v.empty()) { *why = fmt("layer %d seq %d group %d: no attention", l, b, g); return MK_ERR_INVALID_ARG; }
        auto& mv = mrg[b * m.HKV + g];
        std::sort(mv.begin(), mv.end());
        bool ok = !mv.empty();
        for (size_t i = 0; ok && i < mv.size(); ++i) ok = mv[i].first == (int)i && mv[i].second == (int)mv.size();
        if (!ok) { *why = fmt("layer %d seq %d group %d: merge slices do not cover the output once", l, b, g); return MK_ERR_INVALID_ARG; }
      }
  }
  if (m.lm) {
    std::vector<int> rows(m.V, 0);
    for (auto& t : P.tasks) if (t.w[D_OP] == OP_LMHEAD) for (int r = t.w[D_A0]; r < t.w[D_A0] + t.w[D_A1]; ++r) rows[r]++;
    for (int r = 0; r < m.V; ++r) if (rows[r] != 1) { *why = fmt("lm_head row %d written %d times", r, rows[r]); return MK_ERR_INVALID_ARG; }
  }
  (void)nt;
  return MK_OK;
}

// ---- CPU simulation of the persistent loop -------------------------------------------------
// Workers advance through their queues in order; at each event a random worker whose next task's
// waits are satisfied completes it (random interleavings stand in for random latencies). A worker
// told to stall stops before queue position stall_at. If no worker can move while tasks remain,
// the simulated watchdog reports the first blocked wait, as the kernel would.
mk_status simulate_plan(const mk_plan& P, uint64_t seed, int stall_worker, int stall_at, std::string* why) {
  std::mt19937_64 rng(seed);
  std::vector<uint32_t> ctr(P.n_ctr, 0);
  std::vector<int> pos(P.n_workers);
  for (int w = 0; w < P.n_workers; ++w) pos[w] = P.qoff[w];
  int remaining = (int)P.tasks.size();
  auto ready = [&](const Task& t, int* c, uint32_t* tg) {
    for (auto& wt : task_waits(t, P.m.HKV))
      if (wt[0] >= 0 && ctr[wt[0]] < (uint32_t)wt[1]) { *c = wt[0]; *tg = (uint32_t)wt[1]; return false; }
    return true;
  };
  std::vector<int> cand;
  while (remaining > 0) {
    cand.clear();
    for (int w = 0; w < P.n_workers; ++w) {
      if (pos[w] >= P.qoff[w + 1]) continue;
      if (w == stall_worker && pos[w] - P.qoff[w] >= stall_at) continue;
      int c; uint32_t tg;
      if (ready(P.tasks[pos[w]], &c, &tg)) cand.push_back(w);
    }
    if (cand.empty()) {
      for (int w = 0; w < P.n_workers; ++w) {
        if (pos[w] >= P.qoff[w + 1]) continue;
        const Task& t = P.tasks[pos[w]];
        int c = -1; uint32_t tg = 0;
        if (w == stall_worker && pos[w] - P.qoff[w] >= stall_at) {
          if (ready(t, &c, &tg)) continue;   // the stalled worker itself is not blocked by a wait
        }
        if (!ready(t, &c, &tg)) {
          *why = fmt("watchdog: worker %d task %d (op %d, layer %d) waits for counter %d >= %u, observed %u",
                     w, t.w[D_ID], t.w[D_OP], t.w[D_LAYER], c, tg, ctr[c]);
          return MK_ERR_DEVICE;
        }
      }
      *why = fmt("stalled worker %d holds the remaining %d tasks", stall_worker, remaining);
      return MK_ERR_DEVICE;
    }
    const int w = cand[rng() % cand.size()];
    const Task& t = P.tasks[pos[w]];
    if (t.w[D_SIG] >= 0) {
      const uint32_t old = ctr[t.w[D_SIG]]++;
      // last arriver of the router tiles publishes the routing table
      if (t.w[D_SIG2] >= 0 && t.w[D_OP] == OP_ROUTER && old + 1 == (uint32_t)t.w[D_A2]) ctr[t.w[D_SIG2]]++;
    } else if (t.w[D_SIG2] >= 0) {
      ctr[t.w[D_SIG2]]++;
    }
    pos[w]++;
    remaining--;
  }
  return MK_OK;
}

}  // namespace

// ============================================================================== the engine

struct mk_engine {
  mk_model_desc desc;
  Dims m;
  int shape = -1, n_cu = 0, device = 0;
  mk_options opt{};
  LayerPtrs* d_layers = nullptr;
  double* d_inv_freq = nullptr;
  float *d_x = nullptr, *d_qkv = nullptr, *d_rlog = nullptr, *d_h = nullptr, *d_attn = nullptr, *d_apart = nullptr;
  float* d_y = nullptr;
  float* d_o = nullptr;
  uint32_t* d_slot = nullptr;
  RouteTable* d_route = nullptr;
  unsigned long long* d_amax = nullptr;
  uint32_t* d_ctr = nullptr;
  DevError* d_err = nullptr;
  int32_t *d_tasks = nullptr, *d_qoff = nullptr;
  size_t apart_floats = 0, ctr_cap = 0, task_cap = 0, qoff_cap = 0;
  mk_weight_ptrs w{};
  mk_plan* plan = nullptr;
  int steps_since_build = 0;
  int32_t *argmax_out = nullptr, *topk_out = nullptr;
  float* hidden_out = nullptr;
  uint64_t* trace_out = nullptr;
  float* rlog_out = nullptr;
  hipStream_t last_stream = nullptr;
  mk_status sticky = MK_OK;
  std::string msg;
  // chunked prefill's step inputs (allocated at its first call): tokens, positions, lengths
  // [3][max_batch], block tables [max_batch][max_pages], logits [max_batch][V], routed experts
  int32_t *pf_in = nullptr, *pf_bt = nullptr, *pf_topk = nullptr;
  float* pf_logits = nullptr;
};

const mk_model_desc& engine_desc(const mk_engine* e) { return e->desc; }

namespace {

mk_status hip_fail(mk_engine* e, hipError_t err, const char* what) {
  if (e) e->msg = fmt("%s: %s", what, hipGetErrorString(err));
  return MK_ERR_HIP;
}

mk_status hip_ok(mk_engine* e, hipError_t err, const char* what) {
  return err == hipSuccess ? MK_OK : hip_fail(e, err, what);
}

#define HIPCHK(e, call)                                              \
  do {                                                               \
    hipError_t err_ = (call);                                        \
    if (err_ != hipSuccess) return hip_fail((e), err_, #call);       \
  } while (0)

template <class T>
hipError_t dalloc(T** p, size_t n) {
  return hipMalloc(reinterpret_cast<void**>(p), std::max<size_t>(n, 1) * sizeof(T));
}

void free_all(mk_engine* e) {
  void* ps[] = {e->d_layers, e->d_inv_freq, e->d_x, e->d_qkv, e->d_rlog, e->d_h, e->d_y, e->d_o, e->d_slot, e->d_attn, e->d_apart,
                e->d_route, e->d_amax, e->d_ctr, e->d_err, e->d_tasks, e->d_qoff, e->pf_in, e->pf_bt, e->pf_topk,
                e->pf_logits};
  for (void* p : ps) if (p) (void)hipFree(p);
}

}  // namespace

extern "C" {

mk_status mk_create(const mk_model_desc* desc, const mk_weight_ptrs* w, mk_engine** out) {
  std::string why;
  if (!out) return MK_ERR_INVALID_ARG;
  *out = nullptr;
  mk_status st = check_desc(desc, &why);
  if (st != MK_OK) { fprintf(stderr, "mk_create: %s\n", why.c_str()); return st; }
  if (!w || !w->embed || !w->final_norm || !w->attn_norm || !w->w_qkv || !w->w_o || !w->w_router || !w->w_gate ||
      !w->w_up || !w->w_down || !w->k_cache || !w->v_cache || (desc->has_lm_head && !w->lm_head) ||
      (desc->has_router_bias && !w->router_bias)) {
    fprintf(stderr, "mk_create: a required weight pointer is NULL\n");
    return MK_ERR_INVALID_ARG;
  }
  const int L = desc->n_layers;
  for (int l = 0; l < L; ++l)
    if (!w->attn_norm[l] || !w->w_qkv[l] || !w->w_o[l] || !w->w_router[l] || !w->w_gate[l] || !w->w_up[l] ||
        !w->w_down[l] || !w->k_cache[l] || !w->v_cache[l] || (desc->has_router_bias && !w->router_bias[l])) {
      fprintf(stderr, "mk_create: layer %d has a NULL weight pointer\n", l);
      return MK_ERR_INVALID_ARG;
    }
  mk_engine* e = new mk_engine();
  e->desc = *desc;
  e->m = dims_of(*desc);
  e->w = *w;
  e->shape = shape_id(desc->hidden, desc->head_dim, desc->n_q_heads, desc->n_kv_heads, desc->n_experts, desc->top_k,
                      desc->expert_ffn, desc->weight_format);
  e->opt.workers_per_cu = 2;
  e->opt.watchdog_ms = 2000;
  auto fail = [&](mk_status s) { free_all(e); delete e; return s; };
  hipDeviceProp_t prop;
  if (hipGetDevice(&e->device) != hipSuccess || hipGetDeviceProperties(&prop, e->device) != hipSuccess) {
    fprintf(stderr, "mk_create: no HIP device\n");
    return fail(MK_ERR_HIP);
  }
  e->n_cu = prop.multiProcessorCount;
  const Dims& m = e->m;
  std::vector<LayerPtrs> lp(L);
  for (int l = 0; l < L; ++l) {
    lp[l].attn_norm = (const uint16_t*)w->attn_norm[l];
    lp[l].w_qkv = (const uint16_t*)w->w_qkv[l];
    lp[l].w_o = (const uint16_t*)w->w_o[l];
    lp[l].w_router = (const uint16_t*)w->w_router[l];
    lp[l].router_bias = desc->has_router_bias ? w->router_bias[l] : nullptr;
    lp[l].w_gate = (const uint16_t*)w->w_gate[l];
    lp[l].w_up = (const uint16_t*)w->w_up[l];
    lp[l].w_down = (const uint16_t*)w->w_down[l];
    lp[l].k_cache = (uint16_t*)w->k_cache[l];
    lp[l].v_cache = (uint16_t*)w->v_cache[l];
  }
  std::vector<double> inv(m.D / 2);
  for (int i = 0; i < m.D / 2; ++i) inv[i] = std::pow((double)desc->rope_theta, -2.0 * i / m.D);
  bool ok = dalloc(&e->d_layers, L) == hipSuccess && dalloc(&e->d_inv_freq, m.D / 2) == hipSuccess &&
            dalloc(&e->d_x, (size_t)(L + 1) * MAXB * m.H) == hipSuccess &&
            dalloc(&e->d_qkv, (size_t)L * MAXB * m.QKVR) == hipSuccess &&
            dalloc(&e->d_rlog, (size_t)L * MAXB * m.E) == hipSuccess &&
            dalloc(&e->d_h, (size_t)L * MAXB * m.K * m.F) == hipSuccess &&
            dalloc(&e->d_y, (size_t)L * MAXB * m.K * m.H) == hipSuccess &&
            dalloc(&e->d_o, (size_t)L * MAXB * m.H) == hipSuccess &&
            dalloc(&e->d_slot, (size_t)L * MAX_SLOTS * CTR_STRIDE) == hipSuccess &&
            dalloc(&e->d_attn, (size_t)L * MAXB * m.AD) == hipSuccess &&
            dalloc(&e->d_route, (size_t)L) == hipSuccess && dalloc(&e->d_amax, MAXB) == hipSuccess &&
            dalloc(&e->d_err, 1) == hipSuccess;
  if (!ok) { fprintf(stderr, "mk_create: out of device memory\n"); return fail(MK_ERR_OOM); }
  if (hipMemcpy(e->d_layers, lp.data(), sizeof(LayerPtrs) * L, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(e->d_inv_freq, inv.data(), sizeof(double) * inv.size(), hipMemcpyHostToDevice) != hipSuccess ||
      hipMemset(e->d_amax, 0, sizeof(unsigned long long) * MAXB) != hipSuccess ||
      hipMemset(e->d_err, 0, sizeof(DevError)) != hipSuccess ||
      hipMemset(e->d_x, 0, sizeof(float) * (size_t)(L + 1) * MAXB * m.H) != hipSuccess ||
      hipMemset(e->d_slot, 0, sizeof(uint32_t) * (size_t)L * MAX_SLOTS * CTR_STRIDE) != hipSuccess ||
      hipDeviceSynchronize() != hipSuccess) {
    fprintf(stderr, "mk_create: HIP copy failed\n");
    return fail(MK_ERR_HIP);
  }
  *out = e;
  return MK_OK;
}

mk_status mk_set_options(mk_engine* e, const mk_options* o) {
  if (!e || !o) return MK_ERR_INVALID_ARG;
  if (o->workers_per_cu < 0 || o->workers_per_cu > 4 || o->split_keys < 0 || o->watchdog_ms < 0) {
    e->msg = "options out of range";
    return MK_ERR_INVALID_ARG;
  }
  if (o->workers_per_cu) e->opt.workers_per_cu = o->workers_per_cu;
  e->opt.split_keys = o->split_keys;
  if (o->watchdog_ms) e->opt.watchdog_ms = o->watchdog_ms;
  e->opt.flags = o->flags;
  return MK_OK;
}

mk_status mk_build_schedule_chunked(mk_engine* e, int32_t batch, const int32_t* seq_lens_host, int32_t rows_per_seq) {
  if (!e || !seq_lens_host || batch < 1 || batch > e->desc.max_batch || rows_per_seq < 1 || rows_per_seq > batch) {
    if (e) e->msg = "mk_build_schedule: bad batch, seq_lens or rows_per_seq";
    return MK_ERR_INVALID_ARG;
  }
  if (e->desc.weight_format != MK_WEIGHTS_BF16 && batch == 1 && (e->opt.flags & MK_FLAG_OPROJ_PER_GROUP)) {
    e->msg = "mk_build_schedule: MK_FLAG_OPROJ_PER_GROUP (an ablation) exists for bf16 matrices only";
    return MK_ERR_UNSUPPORTED;
  }
  int per_cu = 0;
  HIPCHK(e, step_occupancy(e->shape, batch, step_variant(batch, e->opt.flags, rows_per_seq > 1), &per_cu));
  const int wpc = std::min(e->opt.workers_per_cu, per_cu);
  if (wpc < 1) { e->msg = "kernel does not fit on a CU"; return MK_ERR_UNSUPPORTED; }
  mk_plan* P = new mk_plan();
  std::string why;
  mk_status st = build_plan(e->desc, batch, seq_lens_host, e->n_cu * wpc, e->opt.split_keys, P, &why, e->opt.flags,
                            rows_per_seq);
  if (st == MK_OK) st = validate_plan(*P, &why);
  if (st != MK_OK) { e->msg = "mk_build_schedule: " + why; delete P; return st; }
  // (re)size device buffers that depend on the schedule
  HIPCHK(e, hipDeviceSynchronize());
  const size_t ntask = P->tasks.size(), nq = P->qoff.size(), nctr = P->n_ctr;
  const size_t napart = (size_t)e->m.L * P->parts_per_layer * e->m.PART;
  if (ntask > e->task_cap) { if (e->d_tasks) (void)hipFree(e->d_tasks); e->d_tasks = nullptr; HIPCHK(e, dalloc(&e->d_tasks, ntask * DESC_WORDS)); e->task_cap = ntask; }
  if (nq > e->qoff_cap) { if (e->d_qoff) (void)hipFree(e->d_qoff); e->d_qoff = nullptr; HIPCHK(e, dalloc(&e->d_qoff, nq)); e->qoff_cap = nq; }
  if (nctr > e->ctr_cap) { if (e->d_ctr) (void)hipFree(e->d_ctr); e->d_ctr = nullptr; HIPCHK(e, dalloc(&e->d_ctr, (nctr * CTR_SUB + 1) * CTR_STRIDE)); e->ctr_cap = nctr; }
  if (napart > e->apart_floats) { if (e->d_apart) (void)hipFree(e->d_apart); e->d_apart = nullptr; HIPCHK(e, dalloc(&e->d_apart, napart)); e->apart_floats = napart; }
  HIPCHK(e, hipMemcpy(e->d_tasks, P->tasks.data(), ntask * sizeof(Task), hipMemcpyHostToDevice));
  HIPCHK(e, hipMemcpy(e->d_qoff, P->qoff.data(), nq * sizeof(int32_t), hipMemcpyHostToDevice));
  HIPCHK(e, hipMemset(e->d_ctr, 0, (e->ctr_cap * CTR_SUB + 1) * CTR_STRIDE * sizeof(uint32_t)));
  HIPCHK(e, hipDeviceSynchronize());
  delete e->plan;
  e->plan = P;
  e->steps_since_build = 0;
  return MK_OK;
}

mk_status mk_build_schedule(mk_engine* e, int32_t batch, const int32_t* seq_lens_host) {
  return mk_build_schedule_chunked(e, batch, seq_lens_host, 1);
}

mk_status mk_set_step_outputs(mk_engine* e, int32_t* argmax_out, int32_t* topk_out, float* hidden_out, uint64_t* trace_out,
                              float* router_logits_out) {
  if (!e) return MK_ERR_INVALID_ARG;
  e->argmax_out = argmax_out; e->topk_out = topk_out; e->hidden_out = hidden_out; e->trace_out = trace_out;
  e->rlog_out = router_logits_out;
  return MK_OK;
}

mk_status mk_decode_step(mk_engine* e, const int32_t* tokens, const int32_t* positions, const int32_t* block_tables,
                         const int32_t* seq_lens, float* logits_out, void* stream) {
  if (!e) return MK_ERR_INVALID_ARG;
  if (e->sticky != MK_OK) return e->sticky;
  if (!tokens || !positions || !block_tables || !seq_lens || (e->desc.has_lm_head && !logits_out)) {
    e->msg = "mk_decode_step: NULL input";
    return MK_ERR_INVALID_ARG;
  }
  if (!e->plan) { e->msg = "mk_decode_step: no schedule"; return MK_ERR_NO_SCHEDULE; }
  const mk_plan& P = *e->plan;
  for (int b = 0; b < P.B; ++b)
    if (P.seq_lens[b] + (int64_t)e->steps_since_build * P.rows_per_seq > P.capacity[b]) {
      e->msg = fmt("row %d would reach length %lld, beyond the schedule's capacity %d", b,
                   (long long)(P.seq_lens[b] + (int64_t)e->steps_since_build * P.rows_per_seq), P.capacity[b]);
      return MK_ERR_SCHEDULE_STALE;
    }
  Params p{};
  p.layers = e->d_layers; p.embed = (const uint16_t*)e->w.embed; p.lm_head = (const uint16_t*)e->w.lm_head;
  p.final_norm = (const uint16_t*)e->w.final_norm; p.inv_freq = e->d_inv_freq;
  p.x = e->d_x; p.qkv = e->d_qkv; p.rlog = e->d_rlog; p.route = e->d_route; p.h = e->d_h; p.apart = e->d_apart;
  p.y = e->d_y; p.o = e->d_o; p.slot_ctr = e->d_slot;
  p.attn = e->d_attn; p.amax = e->d_amax; p.ctr = e->d_ctr; p.err = e->d_err;
  p.tasks = e->d_tasks; p.qoff = e->d_qoff;
  p.tokens = tokens; p.positions = positions; p.block_tables = block_tables; p.seq_lens = seq_lens;
  p.logits = e->desc.has_lm_head ? logits_out : nullptr;
  p.argmax_out = e->desc.has_lm_head ? e->argmax_out : nullptr;
  p.topk_out = e->topk_out; p.hidden_out = e->hidden_out; p.rlog_out = e->rlog_out;
  p.trace = (unsigned long long*)e->trace_out;
  p.L = e->m.L; p.V = e->m.V; p.B = P.B; p.max_pages = e->desc.max_pages_per_seq; p.num_pages = e->desc.num_pages;
  p.parts_per_layer = P.parts_per_layer; p.n_workers = P.n_workers; p.n_ctr = P.n_ctr; p.done_ctr = P.done_ctr;
  p.flags = e->opt.flags; p.has_lm_head = e->desc.has_lm_head; p.has_bias = e->desc.has_router_bias;
  p.eps = e->desc.rms_eps;
  p.watchdog_ticks = (uint64_t)e->opt.watchdog_ms * 100000ull;
  hipStream_t st = (hipStream_t)stream;
  size_t lds = 0;
  hipError_t err = launch_step(e->shape, P.B, step_variant(P.B, p.flags, P.rows_per_seq > 1), p, P.n_workers, st, &lds);
  if (err != hipSuccess) return hip_fail(e, err, "cooperative launch");
  e->last_stream = st;
  e->steps_since_build++;
  return MK_OK;
}

static mk_status read_device_error(mk_engine* e) {
  DevError de{};
  HIPCHK(e, hipStreamSynchronize(e->last_stream));
  HIPCHK(e, hipMemcpy(&de, e->d_err, sizeof de, hipMemcpyDeviceToHost));
  if (de.code != DEV_OK) {
    static const char* names[] = {"ok", "dependency wait timed out (watchdog)", "position != seq_len - 1",
                                  "page id out of range", "sequence outgrew its attention split",
                                  "token id out of range", "bad opcode"};
    const char* nm = de.code < 7 ? names[de.code] : "unknown";
    e->msg = fmt("device fault: %s (task %u, worker %u, counter %d, target %u, observed %u, detail %u)", nm, de.task,
                 de.worker, (int)de.counter, de.target, de.observed, de.detail);
    e->sticky = MK_ERR_DEVICE;
    return MK_ERR_DEVICE;
  }
  return MK_OK;
}

mk_status mk_sync(mk_engine* e) {
  if (!e) return MK_ERR_INVALID_ARG;
  if (e->sticky != MK_OK) return e->sticky;
  return read_device_error(e);
}

mk_status mk_get_error(mk_engine* e, char* buf, size_t n) {
  if (!e) { put(buf, n, "NULL engine"); return MK_ERR_INVALID_ARG; }
  mk_status s = e->sticky != MK_OK ? e->sticky : read_device_error(e);
  put(buf, n, e->msg);
  return s;
}

mk_status mk_reset(mk_engine* e) {
  if (!e) return MK_ERR_INVALID_ARG;
  HIPCHK(e, hipDeviceSynchronize());
  HIPCHK(e, hipMemset(e->d_err, 0, sizeof(DevError)));
  if (e->d_ctr) HIPCHK(e, hipMemset(e->d_ctr, 0, (e->ctr_cap * CTR_SUB + 1) * CTR_STRIDE * sizeof(uint32_t)));
  HIPCHK(e, hipMemset(e->d_amax, 0, sizeof(unsigned long long) * MAXB));
  HIPCHK(e, hipMemset(e->d_slot, 0, sizeof(uint32_t) * (size_t)e->m.L * MAX_SLOTS * CTR_STRIDE));
  HIPCHK(e, hipDeviceSynchronize());
  e->sticky = MK_OK;
  e->msg.clear();
  return MK_OK;
}

// ---- chunked prefill ----------------------------------------------------------------------

mk_status mk_prefill(mk_engine* e, const int32_t* tokens_host, int32_t n, int32_t start, const int32_t* block_table_host,
                     float* logits_out, int32_t* topk_out, void* stream) {
  if (!e) return MK_ERR_INVALID_ARG;
  if (e->sticky != MK_OK) return e->sticky;
  const int maxlen = e->desc.max_pages_per_seq * PAGE;
  if (!tokens_host || !block_table_host || n < 1 || start < 0 || (int64_t)start + n > maxlen) {
    e->msg = fmt("mk_prefill: bad arguments (n %d, start %d, longest sequence %d)", n, start, maxlen);
    return MK_ERR_INVALID_ARG;
  }
  for (int i = 0; i < n; ++i)
    if (tokens_host[i] < 0 || tokens_host[i] >= e->desc.vocab) {
      e->msg = fmt("mk_prefill: token %d at %d outside the vocabulary", tokens_host[i], i);
      return MK_ERR_INVALID_ARG;
    }
  const int npages = (int)ceil_div(start + n, PAGE);
  for (int i = 0; i < npages; ++i)
    if (block_table_host[i] < 0 || block_table_host[i] >= e->desc.num_pages) {
      e->msg = fmt("mk_prefill: block table entry %d = %d outside 0..%d", i, block_table_host[i], e->desc.num_pages - 1);
      return MK_ERR_INVALID_ARG;
    }
  const int MB = e->desc.max_batch, MP = e->desc.max_pages_per_seq, L = e->m.L, K = e->m.K;
  const size_t V = (size_t)std::max(1, e->desc.vocab);
  if (!e->pf_in) {
    HIPCHK(e, dalloc(&e->pf_in, 3 * (size_t)MB));
    HIPCHK(e, dalloc(&e->pf_bt, (size_t)MB * MP));
    HIPCHK(e, dalloc(&e->pf_topk, (size_t)L * MB * K));
    HIPCHK(e, dalloc(&e->pf_logits, (size_t)MB * V));
  }
  hipStream_t st = (hipStream_t)stream;
  // every row holds the sequence's block table
  for (int r = 0; r < MB; ++r)
    HIPCHK(e, hipMemcpyAsync(e->pf_bt + (size_t)r * MP, block_table_host, sizeof(int32_t) * npages, hipMemcpyHostToDevice, st));
  // the steps write the routed experts into the prefill's own buffer and nothing else of the caller's
  int32_t* keep_argmax = e->argmax_out; int32_t* keep_topk = e->topk_out; float* keep_hidden = e->hidden_out;
  uint64_t* keep_trace = e->trace_out; float* keep_rlog = e->rlog_out;
  e->argmax_out = nullptr; e->topk_out = topk_out ? e->pf_topk : nullptr; e->hidden_out = nullptr;
  e->trace_out = nullptr; e->rlog_out = nullptr;
  const int R = std::min(MB, n);        // rows per step: consecutive positions of the sequence
  std::vector<int32_t> in(3 * (size_t)MB);
  mk_status stt = MK_OK;
  int built_rows = 0;
  for (int c0 = 0; c0 < n && stt == MK_OK; c0 += R) {
    const int c = std::min(R, n - c0);
    for (int r = 0; r < c; ++r) {
      in[r] = tokens_host[c0 + r];
      in[MB + r] = start + c0 + r;
      in[2 * MB + r] = start + c0 + r + 1;
    }
    if (c != built_rows) {              // (the last chunk may hold fewer rows)
      stt = mk_build_schedule_chunked(e, c, in.data() + 2 * MB, c);
      if (stt != MK_OK) break;
      built_rows = c;
    }
    stt = hip_ok(e, hipMemcpyAsync(e->pf_in, in.data(), sizeof(int32_t) * 3 * MB, hipMemcpyHostToDevice, st), "mk_prefill: copy");
    if (stt != MK_OK) break;
    stt = mk_decode_step(e, e->pf_in, e->pf_in + MB, e->pf_bt, e->pf_in + 2 * MB, e->pf_logits, st);
    if (stt == MK_ERR_SCHEDULE_STALE) {  // the rows outgrew the schedule's attention splits
      stt = mk_build_schedule_chunked(e, c, in.data() + 2 * MB, c);
      if (stt == MK_OK) stt = mk_decode_step(e, e->pf_in, e->pf_in + MB, e->pf_bt, e->pf_in + 2 * MB, e->pf_logits, st);
    }
    if (stt != MK_OK) break;
    if (topk_out)                       // [L][c][K] of this chunk -> rows c0.. of the caller's [L][n][K]
      stt = hip_ok(e, hipMemcpy2DAsync(topk_out + (size_t)c0 * K, sizeof(int32_t) * n * K, e->pf_topk, sizeof(int32_t) * c * K,
                                       sizeof(int32_t) * c * K, L, hipMemcpyDeviceToDevice, st), "mk_prefill: copy");
    if (stt == MK_OK && c0 + c == n && logits_out && e->desc.has_lm_head)
      stt = hip_ok(e, hipMemcpyAsync(logits_out, e->pf_logits + (size_t)(c - 1) * V, sizeof(float) * V,
                                     hipMemcpyDeviceToDevice, st), "mk_prefill: copy");
    // the host staging is rewritten by the next chunk
    if (stt == MK_OK) stt = hip_ok(e, hipStreamSynchronize(st), "mk_prefill: sync");
    if (stt == MK_OK) stt = mk_sync(e);
  }
  e->argmax_out = keep_argmax; e->topk_out = keep_topk; e->hidden_out = keep_hidden;
  e->trace_out = keep_trace; e->rlog_out = keep_rlog;
  // the schedule was the prefill's: the next decode step needs one of its own
  delete e->plan;
  e->plan = nullptr;
  return stt;
}

void mk_destroy(mk_engine* e) {
  if (!e) return;
  (void)hipDeviceSynchronize();
  free_all(e);
  delete e->plan;
  delete e;
}

// ---- measurement helper ------------------------------------------------------------------

mk_status mk_stream_read_bandwidth(const void* buf, size_t bytes, int32_t reps, double* bytes_per_s) {
  if (!buf || bytes < 16 || reps < 1 || !bytes_per_s || ((uintptr_t)buf & 15u)) return MK_ERR_INVALID_ARG;
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return MK_ERR_HIP;
  uint32_t* sink = nullptr;
  hipEvent_t a = nullptr, b = nullptr;
  mk_status st = MK_OK;
  const size_t n16 = bytes / 16;
  const int blocks = 8 * ncu;
  float ms = 0.f;
  if (hipMalloc(&sink, sizeof(uint32_t)) != hipSuccess) return MK_ERR_OOM;
  if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess ||
      launch_stream_read(buf, n16, sink, blocks, nullptr) != hipSuccess ||      // warm-up pass
      hipEventRecord(a, nullptr) != hipSuccess) {
    st = MK_ERR_HIP;
  } else {
    for (int r = 0; r < reps && st == MK_OK; ++r)
      if (launch_stream_read(buf, n16, sink, blocks, nullptr) != hipSuccess) st = MK_ERR_HIP;
    if (st == MK_OK && (hipEventRecord(b, nullptr) != hipSuccess || hipEventSynchronize(b) != hipSuccess ||
                        hipEventElapsedTime(&ms, a, b) != hipSuccess || ms <= 0.f))
      st = MK_ERR_HIP;
  }
  if (st == MK_OK) *bytes_per_s = (double)(n16 * 16) * reps / (ms * 1e-3);
  if (a) (void)hipEventDestroy(a);
  if (b) (void)hipEventDestroy(b);
  (void)hipFree(sink);
  return st;
}

mk_status mk_handoff_litmus(int32_t rounds, int32_t words, int32_t workgroups, uint64_t* stale, uint64_t* checked) {
  if (!stale || !checked || rounds < 1 || rounds > 100000 || words < 1 || words > 65536 || workgroups < 2)
    return MK_ERR_INVALID_ARG;
  int dev = 0, ncu = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      litmus_occupancy(&per_cu) != hipSuccess)
    return MK_ERR_HIP;
  if (workgroups > ncu * per_cu) return MK_ERR_INVALID_ARG;      // every workgroup must be co-resident
  uint32_t *data = nullptr, *ctl = nullptr;
  if (hipMalloc(&data, sizeof(uint32_t) * (size_t)words) != hipSuccess) return MK_ERR_OOM;
  // flag, done and res on lines of their own (256 bytes apart)
  if (hipMalloc(&ctl, 3 * 256) != hipSuccess) { (void)hipFree(data); return MK_ERR_OOM; }
  mk_status st = MK_OK;
  uint32_t res[6] = {0, 0, 0, 0, 0, 0};
  if (hipMemset(data, 0, sizeof(uint32_t) * (size_t)words) != hipSuccess || hipMemset(ctl, 0, 3 * 256) != hipSuccess ||
      launch_litmus(data, ctl, ctl + 64, ctl + 128, rounds, words, workgroups, 100000000ull /* 1 s */, nullptr) != hipSuccess ||
      hipDeviceSynchronize() != hipSuccess || hipMemcpy(res, ctl + 128, sizeof res, hipMemcpyDeviceToHost) != hipSuccess)
    st = MK_ERR_HIP;
  (void)hipFree(data);
  (void)hipFree(ctl);
  if (st != MK_OK) return st;
  *stale = res[0] | ((uint64_t)res[1] << 32);
  *checked = res[2] | ((uint64_t)res[3] << 32);
  if (res[5] != 0 || (int32_t)res[4] != rounds) return MK_ERR_DEVICE;   // a wait hit the watchdog
  return MK_OK;
}

static_assert(LITMUS_SCRATCH_WORDS == MK_LITMUS_NOALLOC_MAX_WORDS, "the scratch array holds the documented maximum");

mk_status mk_handoff_litmus_noalloc(int32_t rounds, int32_t words, int32_t workgroups, uint64_t* stale, uint64_t* checked) {
  if (!stale || !checked || rounds < 1 || rounds > 100000 || words < 1 || workgroups < 2) return MK_ERR_INVALID_ARG;
  if (words > MK_LITMUS_NOALLOC_MAX_WORDS) {
    fprintf(stderr, "mk_handoff_litmus_noalloc: %d words exceed the scratch array's %d\n", words, MK_LITMUS_NOALLOC_MAX_WORDS);
    return MK_ERR_INVALID_ARG;
  }
  int dev = 0, ncu = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      litmus_occupancy(&per_cu) != hipSuccess)
    return MK_ERR_HIP;
  if (workgroups > ncu * per_cu) return MK_ERR_INVALID_ARG;      // every workgroup must be co-resident
  uint32_t* base = nullptr;
  uint32_t res[6] = {0, 0, 0, 0, 0, 0};
  if (litmus_scratch(&base) != hipSuccess ||
      launch_litmus_scratch(base, rounds, words, workgroups, 100000000ull /* 1 s */, nullptr) != hipSuccess ||
      hipStreamSynchronize(nullptr) != hipSuccess ||
      hipMemcpy(res, base + 2 * CTR_STRIDE, sizeof res, hipMemcpyDeviceToHost) != hipSuccess)
    return MK_ERR_HIP;
  *stale = res[0] | ((uint64_t)res[1] << 32);
  *checked = res[2] | ((uint64_t)res[3] << 32);
  if (res[5] != 0 || (int32_t)res[4] != rounds) return MK_ERR_DEVICE;   // a wait hit the watchdog
  return MK_OK;
}

// ---- host-only schedule API ---------------------------------------------------------------

mk_status mk_plan_build(const mk_model_desc* desc, int32_t batch, const int32_t* seq_lens_host, int32_t n_workers,
                        int32_t split_keys, uint32_t flags, int32_t rows_per_seq, mk_plan** out) {
  std::string why;
  if (!out) return MK_ERR_INVALID_ARG;
  *out = nullptr;
  mk_status st = check_desc(desc, &why);
  if (st != MK_OK) { fprintf(stderr, "mk_plan_build: %s\n", why.c_str()); return st; }
  if (!seq_lens_host || batch < 1 || batch > desc->max_batch || n_workers < 1 || split_keys < 0) return MK_ERR_INVALID_ARG;
  mk_plan* P = new mk_plan();
  st = build_plan(*desc, batch, seq_lens_host, n_workers, split_keys, P, &why, (int)flags, rows_per_seq);
  if (st != MK_OK) { fprintf(stderr, "mk_plan_build: %s\n", why.c_str()); delete P; return st; }
  *out = P;
  return MK_OK;
}

mk_status mk_plan_info_get(const mk_plan* P, mk_plan_info* info) {
  if (!P || !info) return MK_ERR_INVALID_ARG;
  info->n_tasks = (int32_t)P->tasks.size();
  info->n_workers = P->n_workers;
  info->n_counters = P->n_ctr;
  info->max_queue = 0;
  std::vector<int64_t> per(P->n_workers, 0);
  for (int w = 0; w < P->n_workers; ++w) {
    info->max_queue = std::max(info->max_queue, P->qoff[w + 1] - P->qoff[w]);
    for (int i = P->qoff[w]; i < P->qoff[w + 1]; ++i) per[w] += P->bytes[i];
  }
  info->bytes_total = std::accumulate(per.begin(), per.end(), (int64_t)0);
  info->bytes_max_worker = *std::max_element(per.begin(), per.end());
  info->n_attn_splits = P->n_attn;
  info->key_capacity_min = *std::min_element(P->capacity.begin(), P->capacity.end());
  info->split_keys = P->split_keys;
  return MK_OK;
}

mk_status mk_plan_export(const mk_plan* P, int32_t* tasks, int32_t* qoff) {
  if (!P) return MK_ERR_INVALID_ARG;
  if (tasks) memcpy(tasks, P->tasks.data(), P->tasks.size() * sizeof(Task));
  if (qoff) memcpy(qoff, P->qoff.data(), P->qoff.size() * sizeof(int32_t));
  return MK_OK;
}

mk_status mk_plan_validate(const mk_plan* P, char* buf, size_t n) {
  if (!P) return MK_ERR_INVALID_ARG;
  std::string why;
  mk_status st = validate_plan(*P, &why);
  put(buf, n, st == MK_OK ? "ok" : why);
  return st;
}

mk_status mk_plan_simulate(const mk_plan* P, uint64_t seed, int32_t stall_worker, int32_t stall_at, char* buf, size_t n) {
  if (!P) return MK_ERR_INVALID_ARG;
  std::string why;
  mk_status st = simulate_plan(*P, seed, stall_worker, stall_at, &why);
  put(buf, n, st == MK_OK ? "ok" : why);
  return st;
}

const mk_plan* mk_engine_plan(const mk_engine* e) { return e ? e->plan : nullptr; }

void mk_plan_destroy(mk_plan* P) { delete P; }

}  // extern "C"
