// Host-visible entry points of the kernel translation unit (mk_kernel.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

#include "../../include/mk.h"
#include "mk_internal.h"

namespace mk {
// 0 = hidden 256 small model, 1 = hidden 2048 30B MoE, plus 2 * weight format (MK_WEIGHTS_*);
// -1 = no compiled instance
int shape_id(int H, int D, int HQ, int HKV, int E, int K, int F, int wf);
// cooperative launch of one step on `grid` workers (batch 1 or up to 8 instance)
// kernel instance for a step: 0 plain, 1 per-KV-group O projection (batch 1 with flag 8), 2 the QKV
// tasks publish the step's K/V (batch > 1 with rows of one sequence in a step)
int step_variant(int batch, int flags, bool kv_first);
hipError_t launch_step(int shape, int batch, int var, const Params& p, int grid, hipStream_t st, size_t* lds_bytes);
hipError_t step_occupancy(int shape, int batch, int var, int* blocks_per_cu);
int split_max();      // keys one attention task may cover
int merge_max();      // attention splits one (sequence, KV group) may have
int out_max_rows();   // rows of one OUT task
int down_rows();      // W_down rows of one queued down item
// plain streaming read of n16 16-byte words on `blocks` workgroups of 256 threads (measurement)
hipError_t launch_stream_read(const void* src, size_t n16, uint32_t* sink, int blocks, hipStream_t st);
// hand-off litmus test (cooperative launch of `grid` workgroups of 256 threads); res[4] as documented
hipError_t launch_litmus(uint32_t* data, uint32_t* flag, uint32_t* done, uint32_t* res, int rounds, int words,
                         int grid, uint64_t wd_ticks, hipStream_t st);
hipError_t litmus_occupancy(int* blocks_per_cu);
// allocation-free form: this device's address of the file-scope scratch array (looked up once per
// device), and a launch that clears its control lines and words with a fill kernel, then runs the test
constexpr int LITMUS_SCRATCH_WORDS = 16384;   // hand-off words the scratch array holds (64 KB)
hipError_t litmus_scratch(uint32_t** base);
hipError_t launch_litmus_scratch(uint32_t* base, int rounds, int words, int grid, uint64_t wd_ticks, hipStream_t st);
}  // namespace mk

// The model description an engine was created with (for the serving loop in mk_server.cpp).
struct mk_engine;
const mk_model_desc& engine_desc(const mk_engine* e);
