/*
 * mk.h - C ABI of libmk, a persistent decode megakernel for AMD MI355X (gfx950).
 *
 * One call to mk_decode_step runs one whole decode step of a parallel-layer MoE transformer for a
 * batch of 1..8 sequences as ONE persistent HIP kernel: resident workgroups pull fixed-size task
 * descriptors from a host-built list in device memory and wait on per-producer counters in HBM
 * instead of kernel boundaries.
 *
 * Sources (cited by page title and section):
 *   P1  aimodeling.com, "cohere-megakernel-north-mini-code-h100": sections "Decode is a bandwidth
 *       game", "One persistent kernel for the whole decode step", "From demo to a full serving
 *       system", "Caveats and takeaways".
 *   P2  "Cohere Megakernel Beats vLLM by 1.58x on H100 GPUs" (latestnews.news), body.
 *   P3  "Cohere Releases Megakernel Engine for North Mini Code, Achieving Up to 1.41x Speedup Over
 *       vLLM" (aibriefing.imbch.dev): "Key Technologies and Architecture", "Scheduling and
 *       Performance Benchmarks", "Limitations and Future Plans".
 *
 * Conventions for every entry point:
 *   - All functions return an mk_status; none throws, aborts or exits. Errors leave the engine
 *     usable unless the status is MK_ERR_DEVICE, which is sticky until mk_reset.
 *   - "device pointer" = memory on the engine's GPU (hipMalloc / torch CUDA tensor storage);
 *     "host pointer" = ordinary process memory. The library never takes ownership of caller memory.
 *   - An engine is not thread-safe: one decode owner thread drives it (P3 "Scheduling and
 *     Performance Benchmarks": a C++ thread owns decode).
 *   - bf16 means IEEE binary32 truncated to its upper 16 bits (stored as uint16).
 */
#ifndef MK_H
#define MK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MK_ABI_VERSION 3
#define MK_MAX_BATCH 8 /* batch sizes up to 8 (P2 body; P3 "Limitations and Future Plans") */

typedef struct mk_engine mk_engine;
typedef struct mk_plan mk_plan;

typedef enum {
  MK_OK = 0,
  MK_ERR_INVALID_ARG = -1,    /* NULL where a pointer is required, sizes out of range        */
  MK_ERR_UNSUPPORTED = -2,    /* a shape with no compiled kernel instance                     */
  MK_ERR_HIP = -3,            /* a HIP runtime call failed (message via mk_get_error)         */
  MK_ERR_OOM = -4,            /* workspace allocation failed                                  */
  MK_ERR_NO_SCHEDULE = -5,    /* mk_decode_step before mk_build_schedule                      */
  MK_ERR_SCHEDULE_STALE = -6, /* sequences outgrew the schedule's key capacity: rebuild it      */
  MK_ERR_DEVICE = -7          /* the kernel reported a fault (watchdog, bad page, bad position) */
} mk_status;

/* Model description. Shapes the library is compiled for:
 *   hidden 256,  heads 8/2 of 32,  8 experts top-2, expert_ffn 128   (small test model)
 *   hidden 2048, heads 32/4 of 128, 128 experts top-8, expert_ffn 768 (30B-total MoE)
 * n_layers, vocab, num_pages, max_pages_per_seq are free; page_size must be 16. */
typedef struct {
  int32_t abi_version;       /* = MK_ABI_VERSION */
  int32_t n_layers;
  int32_t hidden;            /* H */
  int32_t n_q_heads;         /* Hq */
  int32_t n_kv_heads;        /* Hkv (query head h reads KV head h / (Hq/Hkv)) */
  int32_t head_dim;          /* D */
  int32_t n_experts;         /* E */
  int32_t top_k;             /* k experts per token */
  int32_t expert_ffn;        /* F */
  int32_t vocab;             /* V: rows of the embedding table (and of lm_head when present) */
  int32_t page_size;         /* KV tokens per page (16) */
  int32_t num_pages;         /* pages in each layer's K (and V) cache */
  int32_t max_batch;         /* 1..MK_MAX_BATCH */
  int32_t max_pages_per_seq; /* row length of block_tables */
  int32_t has_router_bias;   /* 1: per-layer float32 [E] bias added to router logits */
  int32_t has_lm_head;       /* 0: the step ends at the residual stream (no logits) */
  float rope_theta;          /* RoPE base (rotate-half, full head_dim) */
  float rms_eps;             /* RMSNorm epsilon */
  int32_t weight_format;     /* MK_WEIGHTS_BF16, _FP8 or _MXFP4: the storage of every matrix */
} mk_model_desc;

/* Matrix storage (mk_model_desc.weight_format). The matrices are w_qkv, w_o, w_router, w_gate, w_up,
 * w_down and lm_head; embed, the norm gains and the KV cache are bf16 in every format.
 *   MK_WEIGHTS_BF16  a matrix [R, C] is R rows of C bf16.
 *   MK_WEIGHTS_FP8   FP8 weights (P3 "Limitations and Future Plans": FP8/FP4 megakernels are the
 *                    pages' next step): a matrix [R, C] is R rows of C + 16 bytes - the row's C OCP
 *                    E4M3 codes, then its float32 scale and 12 zero bytes (each row 16-byte aligned);
 *                    weight = E4M3 value of the code * row scale. C must be a multiple of 16.
 *   MK_WEIGHTS_MXFP4 FP4 weights in the OCP microscaling format (MX v1.0 MXFP4): a matrix [R, C] is
 *                    R rows of roundup16(C/2 + C/32) bytes - C/2 bytes of E2M1 codes (element 2i
 *                    in the low nibble of byte i, element 2i + 1 in the high nibble), then the C/32
 *                    E8M0 scale bytes of the row's blocks of 32 elements, then zero bytes; weight =
 *                    E2M1 value of the code * 2^(scale - 127) (scale 255 is NaN). C must be a
 *                    multiple of 32. The per-KV-group O projection flag is refused with FP8 and
 *                    MXFP4 matrices alike. */
#define MK_WEIGHTS_BF16 0
#define MK_WEIGHTS_FP8 1
#define MK_WEIGHTS_MXFP4 2

/* Weight and KV-cache pointers (all device pointers; host arrays of per-layer pointers of length
 * n_layers). Layouts, row-major:
 *   embed [V, H] bf16; lm_head [V, H] bf16 (ignored when has_lm_head = 0); final_norm [H] bf16
 *   attn_norm[l] [H] bf16     the one input norm shared by attention and MoE (parallel layer, P1
 *                             "One persistent kernel for the whole decode step")
 *   w_qkv[l] [(Hq+2Hkv)*D, H] bf16, rows: all q heads, then k heads, then v heads
 *   w_o[l] [H, Hq*D] bf16; w_router[l] [E, H] bf16; router_bias[l] [E] float32 or NULL
 *   w_gate[l], w_up[l] [E, F, H] bf16; w_down[l] [E, H, F] bf16
 *   k_cache[l], v_cache[l] [num_pages, Hkv, page_size, D] bf16 (paged KV, P1 "From demo to a
 *                             full serving system"); written in place by mk_decode_step.
 * The engine keeps the pointers; the caller keeps the memory alive until mk_destroy. */
typedef struct {
  const void* embed;
  const void* lm_head;
  const void* final_norm;
  const void* const* attn_norm;
  const void* const* w_qkv;
  const void* const* w_o;
  const void* const* w_router;
  const float* const* router_bias;
  const void* const* w_gate;
  const void* const* w_up;
  const void* const* w_down;
  void* const* k_cache;
  void* const* v_cache;
} mk_weight_ptrs;

/* Engine tuning knobs (mk_set_options). Zero fields keep their defaults. */
typedef struct {
  int32_t workers_per_cu;    /* resident workgroups per CU (default 2) */
  int32_t split_keys;        /* target keys per attention split (default: chosen from the load) */
  int32_t watchdog_ms;       /* bound on any single dependency wait (default 2000) */
  int32_t flags;             /* MK_FLAG_* */
} mk_options;

#define MK_FLAG_TRACE 1u       /* record per-task timestamps into the trace buffer */
#define MK_FLAG_NO_PREFETCH 2u /* ablation: issue weight loads only after dependencies are met */
/* Ablation: deal the expert slices statically, one (union slot, FFN slice) per task, instead of
 * from the per-layer work queue that tasks drain and steal from (P3 "Scheduling and Performance
 * Benchmarks": dynamic work stealing). Read by mk_build_schedule / mk_plan_build. */
#define MK_FLAG_STATIC_EXPERTS 4u
/* Ablation (batch 1): an output-row task multiplies each KV group's W_o columns as soon as that group's
 * attention merges have landed, instead of after all groups (P1 "One persistent kernel for the whole
 * decode step"). Off by default: measured slower on MI355X. Read by mk_decode_step. */
#define MK_FLAG_OPROJ_PER_GROUP 8u

/* Create an engine for `desc` over caller-owned weights (P1 "One persistent kernel for the whole
 * decode step"). Validates the description, copies the pointer tables to the device and
 * allocates the workspace (activations, partials, counters, task list). Nothing is copied from the
 * weights. Uses the current HIP device. *out is set only on MK_OK. */
mk_status mk_create(const mk_model_desc* desc, const mk_weight_ptrs* weights, mk_engine** out);

/* Set tuning options; takes effect at the next mk_build_schedule. The knobs are the scheduler's:
 * resident workers per CU, attention split length, the bound on a dependency wait, and flags for
 * tracing and ablations (P3 "Scheduling and Performance Benchmarks": mostly static scheduling with
 * dynamic work stealing). MK_ERR_INVALID_ARG for NULL arguments or values out of range
 * (workers_per_cu > 4, negative fields); the engine's options are then unchanged. */
mk_status mk_set_options(mk_engine* e, const mk_options* opt);

/* Build the static task schedule for `batch` sequences whose current lengths (host int32 [batch],
 * counting the token about to be decoded) are seq_lens_host (P3 "Scheduling and Performance
 * Benchmarks": mostly static scheduling). Attention key ranges are split for balance and given
 * room to grow; mk_decode_step returns MK_ERR_SCHEDULE_STALE once any sequence outgrows it.
 * Synchronous; call again when the batch composition changes. */
mk_status mk_build_schedule(mk_engine* e, int32_t batch, const int32_t* seq_lens_host);

/* mk_build_schedule for a batch in which one sequence may hold several rows: consecutive positions
 * of it, one per row, in the same step (chunked prefill, and prefill rows mixed with decode rows:
 * P3 "Limitations and Future Plans" names prefill and mixed batches as the next step for the
 * megakernel). rows_per_seq is the most rows any one sequence holds (1 = mk_build_schedule). With
 * rows_per_seq > 1 the step runs a kernel instance whose QKV tasks write every row's new K/V into
 * the cache before any attention of the layer reads it, so a row sees the keys of the sequence's
 * earlier rows in the same step; rows of one sequence must list the same pages. The host tracks
 * lengths as growing by rows_per_seq per launched step (MK_ERR_SCHEDULE_STALE once a row could
 * outgrow its attention splits). MK_ERR_INVALID_ARG for rows_per_seq outside 1..batch, otherwise as
 * mk_build_schedule. */
mk_status mk_build_schedule_chunked(mk_engine* e, int32_t batch, const int32_t* seq_lens_host,
                                    int32_t rows_per_seq);

/* Prefill through the decode kernel (P2 body: the pages prefill with separate PyTorch kernels; P3
 * "Limitations and Future Plans": prefill in the megakernel is their next step): positions
 * [start, start + n) of ONE sequence, up to max_batch consecutive positions per step, each step
 * built with mk_build_schedule_chunked. Writes the K/V of every position into the pages of
 * block_table_host; K/V of positions < start must already be there. Host arrays (read during the
 * call only): tokens_host int32 [n]; block_table_host int32 [ceil((start + n) / 16)] page ids.
 * Device outputs, caller-owned, NULL = not wanted: logits_out float32 [V] (position start + n - 1),
 * topk_out int32 [L, n, k] (routed experts per layer and position, ascending expert index).
 * Steps run on `stream`; synchronous (returns after the last step). The options, and none of the
 * outputs set by mk_set_step_outputs, apply. On return the engine has no schedule: build one before
 * the next mk_decode_step. MK_ERR_INVALID_ARG (bad sizes, a token outside the vocabulary, a page id
 * outside the cache), MK_ERR_HIP / MK_ERR_DEVICE as mk_decode_step / mk_sync. */
mk_status mk_prefill(mk_engine* e, const int32_t* tokens_host, int32_t n, int32_t start,
                     const int32_t* block_table_host, float* logits_out, int32_t* topk_out, void* stream);

/* Enqueue one decode step on `stream` (a hipStream_t; NULL = default stream): the whole forward
 * pass of every sequence of the batch as ONE kernel launch (P1 "One persistent kernel for the whole
 * decode step"; P3 "Key Technologies and Architecture"), reading the paged KV cache through the
 * block tables (P1 "From demo to a full serving system"). Device pointers, all caller-owned:
 *   tokens int32 [B]                 token being decoded per sequence
 *   positions int32 [B]              its position; must equal seq_lens[b] - 1
 *   block_tables int32 [B, max_pages_per_seq]  page ids; entries past ceil(seq_len/16) unread
 *   seq_lens int32 [B]               context length including the new token
 *   logits_out float32 [B, V]        written (may be NULL when has_lm_head = 0)
 * The new K/V of every sequence is written into the caches at its position before attention.
 * Asynchronous: returns after the launch. Device-side faults surface as MK_ERR_DEVICE from the
 * next mk_decode_step / mk_sync / mk_get_error. Host-side checks, all before anything is launched:
 * MK_ERR_INVALID_ARG (NULL engine or input, NULL logits_out with an lm_head), MK_ERR_NO_SCHEDULE (no
 * mk_build_schedule yet), MK_ERR_SCHEDULE_STALE (a sequence would outgrow the schedule's attention
 * splits: lengths are tracked on the host from the schedule, +1 per launched step; call
 * mk_build_schedule with the current lengths and issue the step again), a sticky MK_ERR_DEVICE. */
mk_status mk_decode_step(mk_engine* e, const int32_t* tokens, const int32_t* positions,
                         const int32_t* block_tables, const int32_t* seq_lens, float* logits_out,
                         void* stream);

/* Optional per-step outputs of the steps launched after this call (device pointers owned by the
 * caller, NULL = off): the greedy token that feeds the next step (the pages' decode benchmark
 * generates its output tokens one step after another, P3 "Scheduling and Performance Benchmarks"),
 * the routed experts of every layer and token (P3 "Key Technologies and Architecture": top-k routed
 * experts), the final residual stream, a per-task trace and the router logits. MK_ERR_INVALID_ARG
 * only for a NULL engine. The pointers must stay valid while steps that write them run.
 *   argmax_out int32 [B]       greedy token (first index of the maximum logit)
 *   topk_out int32 [L, B, k]   routed experts per layer and token, ascending expert index
 *   hidden_out float32 [B, H]  residual stream after the last layer
 *   trace_out uint64 [tasks, 16] when MK_FLAG_TRACE: {task id | worker << 32, t_start, t_ready,
 *                              t_end, mark0..mark11} in 100 MHz ticks (size via mk_plan_info);
 *                              marks are op-specific phase ends, 0 where an op sets none
 *   router_logits_out float32 [L, B, E]  the router logits (bias included) exactly as the routing
 *                              decision of each layer read them */
mk_status mk_set_step_outputs(mk_engine* e, int32_t* argmax_out, int32_t* topk_out,
                              float* hidden_out, uint64_t* trace_out, float* router_logits_out);

/* Wait for the engine's last step (its stream) and report a device fault raised by the kernel
 * (dependency-wait watchdog, bad page id, position != seq_len - 1) as MK_ERR_DEVICE, which stays
 * sticky until mk_reset. The caller is the one thread that owns decode (P3 "Scheduling and
 * Performance Benchmarks": a C++ thread owns the decode loop). MK_ERR_HIP if the runtime fails. */
mk_status mk_sync(mk_engine* e);

/* Describe the last error in `buf` (caller-owned host buffer; NUL-terminated, truncated to n).
 * Synchronizes the engine's last stream to read the device error word, as mk_sync does (the decode
 * owner's view of a failed step, P3 "Scheduling and Performance Benchmarks"). Returns the sticky
 * status (MK_OK if none); with a NULL engine, MK_ERR_INVALID_ARG and "NULL engine" in buf. */
mk_status mk_get_error(mk_engine* e, char* buf, size_t n);

/* Clear a sticky device error and reset every dependency counter and the argmax keys (after
 * MK_ERR_DEVICE). The counters in device memory stand in for kernel boundaries (P1 "One persistent
 * kernel for the whole decode step"); an aborted step leaves them part-way, and the next step needs
 * them at zero. Synchronous (waits for the device). MK_ERR_INVALID_ARG for a NULL engine, MK_ERR_HIP
 * if the runtime fails. */
mk_status mk_reset(mk_engine* e);

/* Release the engine: waits for the device, frees the workspace the engine allocated and the
 * schedule; caller-owned weights, KV cache and step buffers are untouched. NULL is a no-op. Owned,
 * like every other call on the engine, by the one decode thread (P3 "Scheduling and Performance
 * Benchmarks"). */
void mk_destroy(mk_engine* e);

/* Measurement helper: the plain streaming-read bandwidth of the current device, a ceiling to set the
 * step kernel's achieved bandwidth against (decode is bound by HBM bandwidth, P1 "Decode is a
 * bandwidth game"). Reads `bytes` (rounded down to 16) from the device buffer
 * `buf` (16-byte aligned, owned by the caller, not modified) `reps` times with 16-byte non-temporal
 * loads on 8 workgroups per CU, after one untimed pass; *bytes_per_s = bytes read / elapsed time
 * (HIP events on the default stream). Synchronous. MK_ERR_INVALID_ARG for a NULL or misaligned
 * buffer, bytes < 16 or reps < 1; MK_ERR_HIP / MK_ERR_OOM on runtime failures. */
mk_status mk_stream_read_bandwidth(const void* buf, size_t bytes, int32_t reps, double* bytes_per_s);

/* Self-test of the hand-off protocol the step kernel relies on (P1 "One persistent kernel for the
 * whole decode step": tasks hand results to each other through device memory and counters instead of
 * kernel boundaries). `workgroups` co-resident workgroups (cooperative launch; spread over every XCD)
 * run `rounds` rounds; in each, one workgroup writes `words` words with the step kernel's producer
 * sequence (write-through stores, wait for them, barrier, one relaxed counter add) and every other
 * one polls the counter and reads the words with the step kernel's consumer sequence, counting words
 * that do not hold the round's value. *stale = such words over all rounds, *checked = words read.
 * Synchronous; allocates and frees its own small buffers. MK_ERR_INVALID_ARG for NULL outputs,
 * rounds outside 1..100000, words outside 1..65536, or workgroups < 2 or more than can be resident;
 * MK_ERR_DEVICE if a wait exceeded its 1 s bound; MK_ERR_HIP / MK_ERR_OOM on runtime failures. */
mk_status mk_handoff_litmus(int32_t rounds, int32_t words, int32_t workgroups, uint64_t* stale, uint64_t* checked);

/* mk_handoff_litmus for callers that cannot allocate device memory (tight serving loops, harnesses
 * that forbid hipMalloc): the same test and results, with its buffers in a fixed device array that
 * every GPU the library runs on holds until the process ends (the words plus three 256-byte control
 * lines, 64.75 KB); the array is cleared by a fill kernel at every call. It calls no hipMalloc, hipFree
 * or other allocating routine. MK_ERR_INVALID_ARG (and a message on stderr) for words beyond
 * MK_LITMUS_NOALLOC_MAX_WORDS, otherwise the statuses of mk_handoff_litmus. Calls that overlap on one
 * GPU (from several threads, or with work still running on other streams that use it) race on the
 * shared array; the call itself is synchronous on the default stream. */
#define MK_LITMUS_NOALLOC_MAX_WORDS 16384
mk_status mk_handoff_litmus_noalloc(int32_t rounds, int32_t words, int32_t workgroups, uint64_t* stale,
                                    uint64_t* checked);

/* ---- the serving loop's decode owner -------------------------------------------------------
 * A C++ thread that owns an engine and decodes a continuously changing batch (P3 "Scheduling and
 * Performance Benchmarks": a C++ thread owns the decode loop while requests, prefill and batch
 * management run on the control side; P1 "From demo to a full serving system": continuous batching
 * with ragged lengths). A sequence is submitted either with its prefill done elsewhere (K/V of
 * positions [0, prompt_len) already in the pages it owns) or with its prompt, which the owner prefills
 * through the decode kernel: every step, each decoding sequence takes one batch row and the rows left
 * over go to prompt chunks (consecutive positions of one sequence), so prefill and decode share steps
 * (P3 "Limitations and Future Plans": mixed batches are the pages' next step). Up to max_batch
 * sequences are active (admitted at step boundaries, in submission order); a sequence leaves after
 * generating max_new_tokens tokens (greedy: each step's argmax feeds its next step). Whenever the rows'
 * composition changes, the block tables are uploaded and the schedule rebuilt; a sequence that
 * outgrows its attention splits gets the schedule rebuilt too. While a server exists, the engine belongs to its thread: the caller must not call any
 * other function on that engine until mk_server_destroy. Server functions may be called from any one
 * control thread. */
typedef struct mk_server mk_server;

typedef struct {
  int32_t max_batch;          /* rows of the batch, 1..the engine's max_batch */
  int32_t start_held;         /* 1: start with a step budget of 0 (mk_server_run releases steps) */
  int32_t* topk_out;          /* optional device outputs of every step, as in mk_set_step_outputs */
  float* router_logits_out;
  float* hidden_out;
  float* logits_out;          /* optional caller-owned [max_batch, vocab] logits (NULL: the server's own) */
} mk_server_config;

typedef struct {
  int64_t request_id;         /* the caller's id */
  int32_t prompt_len;         /* prompt == NULL: positions already prefilled, decoding starts there;
                                 else: prompt tokens (>= 1) */
  int32_t first_token;        /* prompt == NULL: the token decoded at position prompt_len (else unused) */
  int32_t max_new_tokens;     /* tokens to generate (>= 1) */
  int32_t n_pages;            /* pages the sequence owns, in position order */
  const int32_t* pages;       /* host array, copied at submit; must cover the positions the sequence
                                 will hold: prompt_len + max_new_tokens (prompt: one fewer) */
  const int32_t* prompt;      /* NULL, or the prompt's prompt_len tokens (host, copied at submit): the
                                 owner prefills positions [0, prompt_len - 1) in prompt chunks and decodes
                                 the last prompt token at position prompt_len - 1, whose greedy token is
                                 the first generated one */
} mk_request;

typedef struct {              /* composition of the last step */
  int64_t step;               /* steps run before it */
  int32_t batch;              /* rows */
  int32_t rebuilt;            /* 1 if the schedule was rebuilt for it */
  int64_t request_id[MK_MAX_BATCH];
  int32_t position[MK_MAX_BATCH];
  int32_t token_in[MK_MAX_BATCH];
  int32_t token_out[MK_MAX_BATCH]; /* -1 for a prompt row (it generates nothing) */
  int32_t prefill_rows;       /* rows of the step that were prompt positions */
} mk_server_step;

typedef struct {
  int64_t steps, tokens, rebuilds;  /* tokens: generated ones */
  int32_t active, pending, finished, paused;
  double busy_seconds;        /* wall time the owner spent in steps (schedule rebuilds included) */
  int64_t prefill_tokens;     /* prompt positions the owner prefilled */
} mk_server_stats_t;

/* Start the decode owner over engine e (its step outputs are taken over: argmax by the server, the
 * optional ones from cfg). Allocates the step buffers (device and pinned host) once. MK_ERR_INVALID_ARG
 * for NULL arguments or max_batch outside 1..the engine's max_batch; MK_ERR_OOM / MK_ERR_HIP. */
mk_status mk_server_create(mk_engine* e, const mk_server_config* cfg, mk_server** out);
/* Queue a sequence (copied). MK_ERR_INVALID_ARG for a bad request (page ids outside the pool, too few
 * pages, a token outside the vocabulary, an empty prompt); the server's sticky error if it failed. */
mk_status mk_server_submit(mk_server* s, const mk_request* r);
/* Hold decode between steps and return once the owner is holding (a prefill may then use the GPU and
 * the pages), or the server's sticky error. */
mk_status mk_server_pause(mk_server* s);
mk_status mk_server_resume(mk_server* s);
/* Allow n_steps more steps (-1: no limit; 0: hold after the current step). */
mk_status mk_server_run(mk_server* s, int64_t n_steps);
/* Block until the owner holds: budget used up, paused, or nothing to decode. Returns the sticky error. */
mk_status mk_server_wait(mk_server* s);
/* Finished sequences not yet taken: writes up to max (id, tokens generated) pairs; returns the count,
 * or -1 for bad arguments. */
int32_t mk_server_poll(mk_server* s, int64_t* ids, int32_t* n_tokens, int32_t max);
/* The tokens a finished sequence generated (host buffer of cap); the sequence is then forgotten.
 * MK_ERR_INVALID_ARG if it is unknown, not finished, or cap is too small (*n = tokens needed). */
mk_status mk_server_take(mk_server* s, int64_t request_id, int32_t* tokens, int32_t cap, int32_t* n);
mk_status mk_server_stats(mk_server* s, mk_server_stats_t* out);
/* The last step's composition, and the device address of its logits [batch, vocab] (valid until the
 * next step). */
mk_status mk_server_last_step(mk_server* s, mk_server_step* rec, const float** logits);
/* Describe the owner's first failure (engine status and message) in buf; returns it (MK_OK if none). */
mk_status mk_server_get_error(mk_server* s, char* buf, size_t n);
/* Stop after the current step, join the owner, release the buffers; the engine returns to the caller.
 * Returns the owner's sticky status. */
mk_status mk_server_destroy(mk_server* s);

/* ---- schedule inspection (host only: no GPU needed) -------------------------------------- */
/* The static schedule the host builds for a step (P3 "Scheduling and Performance Benchmarks":
 * mostly static scheduling), inspected, validated and simulated without a GPU. */

typedef struct {
  int32_t n_tasks;           /* descriptors in the step */
  int32_t n_workers;         /* resident workgroups the schedule targets */
  int32_t n_counters;        /* dependency counters */
  int32_t max_queue;         /* longest per-worker queue */
  int64_t bytes_total;       /* weight + KV bytes the tasks stream (cost model) */
  int64_t bytes_max_worker;  /* largest per-worker byte load (cost model) */
  int32_t n_attn_splits;     /* attention split tasks */
  int32_t key_capacity_min;  /* smallest per-sequence key capacity before MK_ERR_SCHEDULE_STALE */
  int32_t split_keys;        /* keys per attention split. Every key past the lengths the schedule was
                              * built for lands in its sequence's open-ended last split, which grows by
                              * one key per step, and that split's length is on the critical path:
                              * rebuilding once a sequence has grown by split_keys / 4 keeps it below
                              * 1.25 x split_keys (the binding and the benchmark do; the serving loop,
                              * which also rebuilds at every change of its batch, at split_keys / 2). */
} mk_plan_info;

/* Build a schedule without any GPU (for validation and tests): same algorithm as
 * mk_build_schedule_chunked for `n_workers` workers; `flags` as in the options struct
 * (MK_FLAG_STATIC_EXPERTS is the one the schedule reads). *out is owned by the caller
 * (mk_plan_destroy). */
mk_status mk_plan_build(const mk_model_desc* desc, int32_t batch, const int32_t* seq_lens_host,
                        int32_t n_workers, int32_t split_keys, uint32_t flags, int32_t rows_per_seq,
                        mk_plan** out);
mk_status mk_plan_info_get(const mk_plan* p, mk_plan_info* info);
/* Copy descriptors (n_tasks x 16 int32) and per-worker queue bounds (n_workers + 1 int32). */
mk_status mk_plan_export(const mk_plan* p, int32_t* tasks, int32_t* queue_offsets);
/* Check the schedule: every task's dependencies are produced by tasks earlier in topological
 * level, counters' targets equal their producer counts, queues are level-ordered (no deadlock
 * with co-resident workers), every output region is written exactly once. Returns MK_OK or
 * MK_ERR_INVALID_ARG with a description in buf. */
mk_status mk_plan_validate(const mk_plan* p, char* buf, size_t n);
/* Discrete-event simulation of the persistent loop on the CPU with random per-task latencies
 * (seeded). Fails (MK_ERR_DEVICE + description) if a dependency wait would never end.
 * stall_worker >= 0 makes that worker stop before its queue position stall_at (a forced stall
 * the simulated watchdog must report). */
mk_status mk_plan_simulate(const mk_plan* p, uint64_t seed, int32_t stall_worker, int32_t stall_at,
                           char* buf, size_t n);
/* Plan of the engine's current schedule (owned by the engine, valid until the next build). */
const mk_plan* mk_engine_plan(const mk_engine* e);
void mk_plan_destroy(mk_plan* p);

#ifdef __cplusplus
}
#endif
#endif /* MK_H */
