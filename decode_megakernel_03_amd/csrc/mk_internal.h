// Internal layouts shared by the host scheduler (mk_host.cpp) and the persistent kernel
// (mk_kernel.hip): task descriptor fields, opcodes, the routing table, the device error word and
// the kernel parameter block. Not part of the public ABI.
#pragma once
#include <stdint.h>

namespace mk {

constexpr int MAXB = 8;          // batch sizes up to 8 (P2 body)
constexpr int PAGE = 16;         // KV tokens per page
constexpr int NT = 256;          // threads per worker (4 wave64s)
constexpr int NWAVE = NT / 64;
constexpr int DESC_WORDS = 16;
// Dependency counters sit 256 bytes apart, one per cache line, so that the pollers and atomics of
// different counters never share a line (and, across lines, spread over memory channels).
constexpr int CTR_STRIDE = 64;      // uint32 between sub-counters (one 256-byte line each)
constexpr int CTR_SUB = 16;         // sub-counters per dependency counter
constexpr int MAX_SLOTS = 64;       // union slots of one layer (at most min(E, K * MAXB))
// Trace record per task (MK_FLAG_TRACE): id | worker << 32, t_start, t_ready, t_end, marks.
constexpr int TRACE_WORDS = 16;
constexpr int TRACE_MARKS = TRACE_WORDS - 4;   // a task descriptor is 16 int32 = 64 bytes

// Task descriptor words. Which a* words an op reads is listed with the opcode.
enum DescWord {
  D_OP = 0, D_LAYER, D_A0, D_A1, D_A2, D_A3, D_A4, D_A5,
  D_W0, D_T0,   // wait until counter[W0] >= T0 (W0 < 0: no wait)
  D_W1, D_T1,   // second wait
  D_SIG,        // counter bumped by one when the task's outputs are visible (< 0: none)
  D_SIG2,       // counter bumped by whoever finishes a multi-task reduction (last arriver)
  D_LEVEL,      // topological level (host validation and trace only)
  D_ID          // task id (trace only)
};

// Opcodes. One parallel layer is QKV/ROUTER -> GATEUP/ATTN -> OUT (P1 "One persistent kernel
// for the whole decode step": attention and MoE read the same normed input; the residual add
// rejoins them). LMHEAD follows the last layer.
enum Op {
  OP_NOP = 0,
  OP_QKV = 1,     // a0 row0, a1 nrows: qkv[l][b][row] = W_qkv[row] . rmsnorm(x_l[b])
  OP_ROUTER = 2,  // a0 row0, a1 nrows, a2 router tiles: logits; the last tile routes (top-k)
  OP_GATEUP = 3,  // static: a0 union slot, a1 f0, a2 nf, a3 -1: h = SiLU(W_gate n) * (W_up n) on rows f0..
                  // queue: a0 own sub-queue, a1 sub-queues, a2 slices per slot, a3 queue counter,
                  // a4 rows per slice, a5 down items per slot (0: none) | O-projection items << 16:
                  // the layer's work queue holds every (slot, slice) gate/up item, then the
                  // O-projection row blocks (they wait on the attention counter, which is the queue
                  // counter - 1; bf16 and MXFP4 matrices), then every (slot, row block) down item
  OP_ATTN = 4,    // a0 b, a1 g, a2 k0, a3 k1 (-1 = to seq_len, the split holding the new token),
                  // a4 first partial of (b, g) in the layer, a5 split | nsplit << 16
  OP_OUT = 5,     // a0 row0, a1 nrows, a2 attention counter (KV group g's merges on sub-counters
                  // g*CTR_SUB/HKV ..), a3 its target, a4 bits: 1 = the down projections come from the
                  // queued down items (y): x_{l+1} = x_l + W_o attn + sum_i w_i W_down[e_i] h_i;
                  // 4 = the O projection comes from the queued O-projection items (o) as well
  OP_LMHEAD = 6,  // a0 row0, a1 nrows: logits + running argmax
  OP_MERGE = 7,   // a0 b, a1 g, a2 slice, a3 slices, a4 first partial, a5 nsplit: attention output
  OP_COUNT
};

// Routing decision of one layer, written by the last router tile (sc1 stores), read by GATEUP
// and OUT. Selected experts are kept in ascending expert index (the MoE sum order).
struct RouteTable {
  int32_t n_union;                 // distinct experts over the batch
  int32_t pad[3];
  int32_t union_e[64];             // ascending expert ids
  int32_t n_tok[64];               // tokens routed to union slot u
  int32_t tok_bi[64][MAXB];        // (b << 8) | i : token b's i-th selected expert is union_e[u]
  int32_t sel[MAXB][8];            // token b's selected experts, ascending
  float w[MAXB][8];                // their softmax weights
};

// Sticky device error (first fault wins), read by the host after a step.
enum DevErr : uint32_t {
  DEV_OK = 0, DEV_TIMEOUT = 1, DEV_BAD_POS = 2, DEV_BAD_PAGE = 3, DEV_STALE = 4, DEV_BAD_TOKEN = 5,
  DEV_BAD_OP = 6
};
struct DevError {
  uint32_t code, task, worker, counter, target, observed, detail, abort_flag;
};

struct LayerPtrs {
  const uint16_t* attn_norm;
  const uint16_t* w_qkv;
  const uint16_t* w_o;
  const uint16_t* w_router;
  const float* router_bias;
  const uint16_t* w_gate;
  const uint16_t* w_up;
  const uint16_t* w_down;
  uint16_t* k_cache;
  uint16_t* v_cache;
};

struct Params {
  const LayerPtrs* layers;   // [L]
  const uint16_t* embed;
  const uint16_t* lm_head;
  const uint16_t* final_norm;
  const double* inv_freq;    // [D/2] theta^(-2i/D), float64

  float* x;                  // [L+1][MAXB][H] residual stream (x[0] unused: layer 0 reads embed)
  float* qkv;                // [L][MAXB][QKVR]
  float* rlog;               // [L][MAXB][E]
  RouteTable* route;         // [L]
  float* h;                  // [L][MAXB][K][F]
  float* y;                  // [L][MAXB][K][H] down projection of token b's i-th expert (queued down items)
  float* o;                  // [L][MAXB][H] O projection of token b's attention (queued O-projection items)
  uint32_t* slot_ctr;        // [L][64] lines of CTR_STRIDE: gate/up items done per union slot (zeroed per step)
  float* apart;              // [L][parts_per_layer][HPG * (D + 2)]
  float* attn;               // [L][MAXB][HQ * D]
  unsigned long long* amax;  // [MAXB] packed (ordered logit << 32 | ~index)
  uint32_t* ctr;             // [n_ctr][CTR_SUB] + 1 lines of CTR_STRIDE: dependency counters (zero between steps)
  DevError* err;

  const int32_t* tasks;      // [n_tasks][16]
  const int32_t* qoff;       // [n_workers + 1]

  const int32_t* tokens;
  const int32_t* positions;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  float* logits;             // [B][V] or null
  int32_t* argmax_out;       // [B] or null
  int32_t* topk_out;         // [L][B][K] or null
  float* hidden_out;         // [B][H] or null
  float* rlog_out;           // [L][B][E] or null
  unsigned long long* trace; // [n_tasks][4] or null

  int32_t L, V, B, max_pages, num_pages, parts_per_layer, n_workers, n_ctr;
  int32_t done_ctr;          // counter index used for end-of-step detection
  int32_t flags, has_lm_head, has_bias;
  float eps;
  uint64_t watchdog_ticks;   // 100 MHz ticks
};

}  // namespace mk
