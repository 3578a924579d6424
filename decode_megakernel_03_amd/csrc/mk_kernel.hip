// The persistent decode megakernel for gfx950 (MI355X).
//
// One launch runs a whole decode step (P1 "One persistent kernel for the whole decode step"):
// every resident workgroup ("worker", 256 threads = 4 wave64s; two per CU) walks its own queue of
// 64-byte task descriptors built by the host (P3 "Key Technologies and Architecture": a task list
// in global memory), waits on per-producer counters in HBM instead of kernel boundaries, runs the
// task and bumps the counter of what it produced.
//
// Hand-off protocol (measured on MI355X: an agent-scope release fence writes back the whole L2 and
// costs ~12 us inside a streaming loop, so it is never used):
//   producer: outputs written with sc1 (agent-coherent, write-through) buffer stores;
//             s_waitcnt vmcnt(0) in every wave; workgroup barrier; one relaxed atomic add.
//   consumer: thread 0 polls the counter with relaxed agent-scope loads (s_sleep backoff, bounded
//             by a watchdog); workgroup barrier; hand-off data read with sc1 buffer loads.
// Weights are activation-independent, so each task issues its first block of weight loads BEFORE
// waiting on its dependencies (P1: weights stream while the producers finish).
//
// Numerics: activations stay float32 everywhere; dot products use explicit fmaf in a fixed order;
// no float atomics, so a step is bitwise deterministic whatever the timing. The file is compiled
// with -ffp-contract=off so that the non-dot arithmetic rounds exactly as written.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "mk_internal.h"
#include "mk_launch.h"

namespace mk {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

template <int H_, int D_, int HQ_, int HKV_, int E_, int K_, int F_, int WF_ = 0>
struct Shape {
  static constexpr int H = H_, D = D_, HQ = HQ_, HKV = HKV_, E = E_, K = K_, F = F_;
  // matrices (QKV, O, router, experts, lm_head): 0 bf16 rows; 1 FP8 rows (OCP E4M3 codes, then the
  // row's float32 scale in a 16-byte tail); 2 MXFP4 rows (E2M1 codes two to a byte, then one E8M0
  // scale byte per block of 32 inputs, padded to 16 bytes). P3 "Limitations and Future Plans" names
  // FP8/FP4 kernels as the next step. kw(k): 16-bit words of codes in a row of k inputs; rw(k): the
  // row's stride in 16-bit words.
  static constexpr int WF = WF_;
  static constexpr int kw(int k) { return WF == 2 ? k / 4 : WF == 1 ? k / 2 : k; }
  static constexpr int rw(int k) { return WF == 2 ? (k / 2 + k / 32 + 15) / 16 * 8 : WF == 1 ? k / 2 + 8 : k; }
  static constexpr int HPG = HQ / HKV;           // query heads per KV head (GQA group)
  static constexpr int QKVR = (HQ + 2 * HKV) * D;
  static constexpr int AD = HQ * D;              // attention output width
  static constexpr int PART = HPG * (D + 2);     // one attention partial: m[HPG] l[HPG] o[HPG][D]
};
using ShapeSmall = Shape<256, 32, 8, 2, 8, 2, 128>;
using ShapeFull = Shape<2048, 128, 32, 4, 128, 8, 768>;
using ShapeSmall8 = Shape<256, 32, 8, 2, 8, 2, 128, 1>;
using ShapeFull8 = Shape<2048, 128, 32, 4, 128, 8, 768, 1>;
using ShapeSmall4 = Shape<256, 32, 8, 2, 8, 2, 128, 2>;
using ShapeFull4 = Shape<2048, 128, 32, 4, 128, 8, 768, 2>;

constexpr int SPLIT_MAX = 1024;   // keys one attention task may cover (LDS score buffer)
constexpr int MERGE_MAX = (SPLIT_MAX + 1) / 2;   // splits one (sequence, KV group) may have
constexpr int OUT_MAXR = 5;       // most rows of one OUT task
constexpr int OUT_OT = 4;         // tokens whose attention vectors an OUT task stages together
constexpr int DOWN_ROWS = 128;    // W_down rows of one queued down item (192 KB of the full-size expert)
constexpr int STEAL_PROBES = 4;   // sub-queues an expert task draws from (its own, then 3 more)
constexpr int SC1 = 16;           // buffer cache-policy bit for agent-coherent access

// ------------------------------------------------------------------------------ primitives

// Every op is a separate (non-inlined) function so that registers are allocated per op. They reach
// the kernel parameters through the kernarg segment pointer (scalar loads) and use file-scope LDS.
extern __shared__ __align__(16) float smem[];
typedef const __attribute__((address_space(4))) Params CParams;

__device__ __forceinline__ CParams& P() {
#if defined(__HIP_DEVICE_COMPILE__)
  // laundered so that each op re-reads its parameters instead of keeping them live across ops
  uint64_t a = reinterpret_cast<uint64_t>(__builtin_amdgcn_kernarg_segment_ptr());
  asm volatile("" : "+s"(a));
  return *reinterpret_cast<CParams*>(a);
#else
  return *reinterpret_cast<CParams*>(0);
#endif
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7FFFFFFF, 0x00020000);
}
__device__ __forceinline__ float ldc(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, SC1));
}
__device__ __forceinline__ int32_t ldci(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(int32_t, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, SC1));
}
__device__ __forceinline__ f4 ldc4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, SC1));
}
__device__ __forceinline__ void stc(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, SC1);
}
__device__ __forceinline__ void stci(__amdgpu_buffer_rsrc_t r, uint32_t off, int32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, SC1);
}
__device__ __forceinline__ void stc4(__amdgpu_buffer_rsrc_t r, uint32_t off, f4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), r, off, 0, SC1);
}
typedef const __attribute__((address_space(1))) u4 gu4;
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lv4s;     // LDS pointer for the transpose reads

// Step-constant tables (descriptors, queue bounds, layer pointers, per-step inputs) are read
// through the constant address space so that uniform reads become scalar loads.
template <class T>
__device__ __forceinline__ const __attribute__((address_space(4))) T* cst(const T* p) {
  return (const __attribute__((address_space(4))) T*)p;
}
__device__ __forceinline__ u4 ldw(const void* p) {   // streamed weight / KV load (global memory)
  return __builtin_nontemporal_load((gu4*)p);
}
__device__ __forceinline__ uint32_t ctr_load(const uint32_t* c) {
  return __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ctr_add(uint32_t* c, uint32_t v) {
  return __hip_atomic_fetch_add(c, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void drain() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// threadIdx.x made opaque per call, so that per-lane values derived from it are recomputed inside
// each task instead of being hoisted out of the task loop into long-lived (spilled) registers
__device__ __forceinline__ int tid() {
  int x = (int)threadIdx.x;
  asm volatile("" : "+v"(x));
  return x;
}
__device__ __forceinline__ uint64_t now() { return __builtin_amdgcn_s_memrealtime(); }

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf1(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
__device__ __forceinline__ uint32_t f2bf(float f) {   // round to nearest even (NaN stays quiet NaN)
  const uint32_t u = __float_as_uint(f);
  const uint32_t r = ((u + 0x7fffu + ((u >> 16) & 1u)) >> 16) & 0xffffu;
  const uint32_t q = ((u >> 16) | 0x40u) & 0xffffu;
  return (u & 0x7fffffffu) > 0x7f800000u ? q : r;
}

// acc += sum_m w[m] * a[m] over the 8 bf16 of w, in element order
__device__ __forceinline__ float dot8(u4 w, f4 a0, f4 a1, float acc) {
  acc = __builtin_fmaf(bf_lo(w.x), a0.x, acc);
  acc = __builtin_fmaf(bf_hi(w.x), a0.y, acc);
  acc = __builtin_fmaf(bf_lo(w.y), a0.z, acc);
  acc = __builtin_fmaf(bf_hi(w.y), a0.w, acc);
  acc = __builtin_fmaf(bf_lo(w.z), a1.x, acc);
  acc = __builtin_fmaf(bf_hi(w.z), a1.y, acc);
  acc = __builtin_fmaf(bf_lo(w.w), a1.z, acc);
  acc = __builtin_fmaf(bf_hi(w.w), a1.w, acc);
  return acc;
}

// Value of an E8M0 scale byte: 2^(e - 127); e = 0 is the subnormal 2^-127, e = 255 NaN
__device__ __forceinline__ float e8m0(uint32_t e) {
  return __uint_as_float(e == 255u ? 0x7fc00000u : e ? e << 23 : 0x00400000u);
}

// acc += sum_m w[m] * a[m] over the 16 E4M3 codes of w (bytes in element order), in element order;
// the hardware conversion takes two codes of a 16-bit half at a time
typedef float f2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot16e4m3(u4 w, f4 a0, f4 a1, f4 a2, f4 a3, float acc) {
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
  const f4 a[4] = {a0, a1, a2, a3};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const f2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(wd[k], false), hi = __builtin_amdgcn_cvt_pk_f32_fp8(wd[k], true);
    acc = __builtin_fmaf(lo.x, a[k].x, acc);
    acc = __builtin_fmaf(lo.y, a[k].y, acc);
    acc = __builtin_fmaf(hi.x, a[k].z, acc);
    acc = __builtin_fmaf(hi.y, a[k].w, acc);
  }
  return acc;
}

// The 8 E2M1 codes of a dword (element 2i in the low nibble of byte i) times the block scale s (a
// power of two, so every product is exact in the normal range), in element order
struct f8v { float v[8]; };
__device__ __forceinline__ f8v dec8e2m1(uint32_t w, float s) {
  const f2 b0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 0);
  const f2 b1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 1);
  const f2 b2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 2);
  const f2 b3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 3);
  return f8v{{b0.x, b0.y, b1.x, b1.y, b2.x, b2.y, b3.x, b3.y}};
}

// acc += sum_m w[m] * a[m] over 8 decoded weights and 8 activations, in element order
__device__ __forceinline__ float dot8f(const f8v& w, f4 a0, f4 a1, float acc) {
  acc = __builtin_fmaf(w.v[0], a0.x, acc);
  acc = __builtin_fmaf(w.v[1], a0.y, acc);
  acc = __builtin_fmaf(w.v[2], a0.z, acc);
  acc = __builtin_fmaf(w.v[3], a0.w, acc);
  acc = __builtin_fmaf(w.v[4], a1.x, acc);
  acc = __builtin_fmaf(w.v[5], a1.y, acc);
  acc = __builtin_fmaf(w.v[6], a1.z, acc);
  acc = __builtin_fmaf(w.v[7], a1.w, acc);
  return acc;
}

// Value of `v` in a partner lane within the same 16-lane row, by DPP (no LDS traffic). For a bit b
// of the lane index (b = 1, 2, 4, 8) the partner differs from the lane exactly in that bit's half:
// quad permutes for 1 and 2, the half-row mirror (i <-> 7 - i) for 4, the row mirror (i <-> 15 - i)
// for 8. Either partner pattern serves sums and half-exchanging reductions alike.
template <int BIT>
__device__ __forceinline__ float dpp_partner(float v) {
  constexpr int ctrl = BIT == 1 ? 0xB1 : BIT == 2 ? 0x4E : BIT == 4 ? 0x141 : 0x140;
  static_assert(BIT == 1 || BIT == 2 || BIT == 4 || BIT == 8, "");
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float partner(float v, int bit) {   // any bit of the lane index
  switch (bit) {
    case 1: return dpp_partner<1>(v);
    case 2: return dpp_partner<2>(v);
    case 4: return dpp_partner<4>(v);
    case 8: return dpp_partner<8>(v);
    case 16:   // swizzle in bit-mask mode: source lane = lane ^ 16 within each 32-lane half
      return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
    default: return __shfl_xor(v, bit, 64);
  }
}
__device__ __forceinline__ float lane_val(float v, int l) {     // v of lane l (uniform l)
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// Reductions over aligned groups of N lanes; for N = 64 the wave must be fully active (the last
// step reads lanes 0 and 32) and the result is the same in every lane.
template <int N>
__device__ __forceinline__ float wsum(float v) {
#pragma unroll
  for (int m = 1; m < N && m < 32; m <<= 1) v += partner(v, m);
  if constexpr (N == 64) v = lane_val(v, 0) + lane_val(v, 32);
  return v;
}
template <int N>
__device__ __forceinline__ float wmax(float v) {
#pragma unroll
  for (int m = 1; m < N && m < 32; m <<= 1) v = fmaxf(v, partner(v, m));
  if constexpr (N == 64) v = fmaxf(lane_val(v, 0), lane_val(v, 32));
  return v;
}

// ------------------------------------------------------------------------------ control

struct Ctl {            // small per-worker control block in static LDS
  int ok;
  int flag;
  int item;             // expert-queue draw broadcast to the workgroup
  int steal;            // sub-queue to steal from next (-1: none had items left)
  int norm_l;           // layer whose normed input the expert-slice staging area holds (-1: none)
  unsigned long long t_ready;   // when the task's last dependency wait ended (trace)
  unsigned long long mark[TRACE_MARKS];   // op-specific phase ends (trace)
  int toks[MAXB];       // batch rows of the tokens a task works on
  int trank[MAXB];      // rank of an expert in each listed token's selection (expert slices)
  unsigned long long mask[MAXB][2];   // per token: experts selected by the router (bit e)
  alignas(16) RouteTable rt;   // the layer's routing decision, copied in one round trip
};
__shared__ Ctl ctl_s;
static_assert(sizeof(RouteTable) % 16 == 0, "");

// Trace: time the end of an op's phase i (0..3); no-op unless tracing.
// The latest of the four waves counts: each wave's first lane folds its clock into an LDS max.
#define MARK(i) do { if ((p.flags & 1) && (tid() & 63) == 0) atomicMax(&ctl_s.mark[i], (unsigned long long)now()); } while (0)

// Copy layer l's routing table into LDS: every thread loads 16 bytes, one round trip.
__device__ __forceinline__ void load_route(CParams& p, int l) {
  const __amdgpu_buffer_rsrc_t R = rsrc(p.route + l);
  f4* dst = reinterpret_cast<f4*>(&ctl_s.rt);
  for (int i = tid(); i < (int)(sizeof(RouteTable) / 16); i += NT) dst[i] = ldc4(R, 16u * i);
  __syncthreads();
}

__device__ void raise_error(CParams& p, uint32_t code, int task, int ctr, uint32_t target,
                            uint32_t observed, uint32_t detail) {
  uint32_t prev = atomicCAS(&p.err->code, 0u, code);
  if (prev == 0) {
    __hip_atomic_store(&p.err->task, (uint32_t)task, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&p.err->worker, (uint32_t)blockIdx.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&p.err->counter, (uint32_t)ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&p.err->target, target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&p.err->observed, observed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&p.err->detail, detail, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __hip_atomic_store(&p.err->abort_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Each dependency counter is CTR_SUB sub-counters on lines of their own: a signal adds to its
// worker's sub-counter and a wait sums them. Atomics to one address complete one after another
// (tens of ns each), so a burst of several hundred signals on one line delays the last of them by
// microseconds; spread over CTR_SUB lines the burst drains CTR_SUB times faster.
__device__ __forceinline__ uint32_t* ctr_at(CParams& p, int c, int s) {
  return p.ctr + ((size_t)c * CTR_SUB + s) * CTR_STRIDE;
}

// Sum of counter c's sub-counters, one load per lane of the calling wave (wave-uniform result).
__device__ __forceinline__ uint32_t ctr_sum(CParams& p, int c, int lane) {
  const uint32_t v = lane < CTR_SUB ? ctr_load(ctr_at(p, c, lane)) : 0u;
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < CTR_SUB; ++i) s += __builtin_amdgcn_readlane(v, i);
  return s;
}

// Block until counter c >= target (wave 0 polls, the workgroup waits at a barrier). Returns false
// if the step was aborted or this wait exceeded the watchdog (which then aborts the step).
__device__ __forceinline__ bool wait_ge(CParams& p, Ctl& ctl, int c, uint32_t target, int task) {
  if (c < 0) return true;
  const int tx = tid(), lane = tx & 63;
  if (__builtin_amdgcn_readfirstlane(tx >> 6) == 0) {
    int ok = 1;
    const bool tr = p.flags & 1;
    uint64_t q0 = tr ? now() : 0;
    uint32_t v = ctr_sum(p, c, lane);
    if (tr && lane == 0) {   // trace: round trip of the first and of the last poll, and the number of polls
      const uint64_t q1 = now();
      ctl.mark[8] = q1 - q0;
      ctl.mark[10] = q1 - q0;
      ctl.mark[11] = 1;
    }
    if (v < target) {
      const uint64_t t0 = now();
      uint32_t it = 0;
      for (;;) {
        __builtin_amdgcn_s_sleep(1);
        if (tr) q0 = now();
        v = ctr_sum(p, c, lane);
        if (tr && lane == 0) { ctl.mark[10] = now() - q0; ctl.mark[11] += 1; }
        if (v >= target) break;
        if ((++it & 15u) == 0) {
          if (__builtin_amdgcn_readfirstlane(ctr_load(&p.err->abort_flag))) { ok = 0; break; }
          if (now() - t0 > p.watchdog_ticks) {
            if (lane == 0) raise_error(p, DEV_TIMEOUT, task, c, target, v, 0);
            ok = 0;
            break;
          }
        }
      }
    }
    if (lane == 0) {
      ctl.ok = ok;
      ctl.t_ready = now();
    }
  }
  __syncthreads();
  const bool ok = ctl.ok != 0;
  __syncthreads();
  return ok;
}

// Block until the single word *w (a union slot's count of finished gate/up items) reaches target
// (wave 0 polls, the workgroup waits at a barrier). False if the step was aborted or the watchdog fired.
__device__ __forceinline__ bool wait_word(CParams& p, Ctl& ctl, const uint32_t* w, uint32_t target, int task, uint32_t detail) {
  const int tx = tid(), lane = tx & 63;
  if (__builtin_amdgcn_readfirstlane(tx >> 6) == 0) {
    int ok = 1;
    uint32_t v = __builtin_amdgcn_readfirstlane(ctr_load(w));
    if (v < target) {
      const uint64_t t0 = now();
      uint32_t it = 0;
      for (;;) {
        __builtin_amdgcn_s_sleep(1);
        v = __builtin_amdgcn_readfirstlane(ctr_load(w));
        if (v >= target) break;
        if ((++it & 15u) == 0) {
          if (__builtin_amdgcn_readfirstlane(ctr_load(&p.err->abort_flag))) { ok = 0; break; }
          if (now() - t0 > p.watchdog_ticks) {
            if (lane == 0) raise_error(p, DEV_TIMEOUT, task, -1, target, v, detail);
            ok = 0;
            break;
          }
        }
      }
    }
    if (lane == 0) {
      ctl.ok = ok;
      ctl.t_ready = now();
    }
  }
  __syncthreads();
  const bool ok = ctl.ok != 0;
  __syncthreads();
  return ok;
}

// Block until counter c0 >= t0 and counter c1 >= t1, polling both in the same round trip.
__device__ __forceinline__ bool wait_ge2(CParams& p, Ctl& ctl, int c0, uint32_t t0, int c1, uint32_t t1, int task) {
  const int tx = tid(), lane = tx & 63;
  if (__builtin_amdgcn_readfirstlane(tx >> 6) == 0) {
    int ok = 1;
    uint32_t v0 = c0 >= 0 ? ctr_sum(p, c0, lane) : t0, v1 = c1 >= 0 ? ctr_sum(p, c1, lane) : t1;
    if (v0 < t0 || v1 < t1) {
      const uint64_t ts = now();
      uint32_t it = 0;
      for (;;) {
        __builtin_amdgcn_s_sleep(1);
        if (c0 >= 0) v0 = ctr_sum(p, c0, lane);
        if (c1 >= 0) v1 = ctr_sum(p, c1, lane);
        if (v0 >= t0 && v1 >= t1) break;
        if ((++it & 15u) == 0) {
          if (__builtin_amdgcn_readfirstlane(ctr_load(&p.err->abort_flag))) { ok = 0; break; }
          if (now() - ts > p.watchdog_ticks) {
            const bool first = v0 < t0;
            if (lane == 0) raise_error(p, DEV_TIMEOUT, task, first ? c0 : c1, first ? t0 : t1, first ? v0 : v1, 0);
            ok = 0;
            break;
          }
        }
      }
    }
    if (lane == 0) {
      ctl.ok = ok;
      ctl.t_ready = now();
    }
  }
  __syncthreads();
  const bool ok = ctl.ok != 0;
  __syncthreads();
  return ok;
}

// Make this worker's sc1 stores visible, then bump counter c. Returns the counter's old value
// (meaningful on thread 0 only; broadcast through ctl.flag when `want_old`).
// drain() that, when tracing, records how long wave 0 waited
__device__ __forceinline__ void drain_t(CParams& p) {
  if ((p.flags & 1) && tid() == 0) {
    const uint64_t d0 = now();
    drain();
    ctl_s.mark[9] = now() - d0;
  }
  drain();
}

// A signal adds to its worker's sub-counter (waits sum all CTR_SUB). A signal whose old value is used
// counts on sub-counter 0 only (all of that counter's signals do), so that the old value is the
// number of earlier signals. A signal of group `grp` >= 0 (of the attention counter's HKV groups)
// adds to one of that group's CTR_SUB / HKV sub-counters, so that a waiter can count each group.
template <int HKV = 1>
__device__ __forceinline__ uint32_t signal(CParams& p, Ctl& ctl, int c, bool want_old, int grp = -1) {
  drain();
  __syncthreads();
  uint32_t old = 0;
  if (tid() == 0 && c >= 0) {
    constexpr int per = CTR_SUB / HKV;
    const int sub = want_old ? 0 : grp >= 0 ? grp * per + (int)(blockIdx.x % per) : (int)(blockIdx.x % CTR_SUB);
    old = ctr_add(ctr_at(p, c, sub), 1u);
    if (want_old) ctl.flag = (int)old;
  }
  if (want_old) {
    __syncthreads();
    old = (uint32_t)ctl.flag;
    __syncthreads();
  }
  return old;
}

__device__ __forceinline__ bool aborted(CParams& p) { return ctr_load(&p.err->abort_flag) != 0; }

// ------------------------------------------------------------------------------ GEMV engine
//
// A wave multiplies rows of a bf16 matrix (row length KD) with float32 activations held in LDS.
// LPR lanes cover one row; each lane owns CPL 16-byte chunks of the row (chunk lir + j*LPR), so
// every load instruction of a wave reads whole contiguous row segments. A "pass" is RPP rows;
// passes are dealt round-robin to the 4 waves; a "block" is NP passes per wave, double-buffered in
// registers so the next block's loads are in flight while the current one is multiplied.

template <int KD>
struct Geo {
  static constexpr int CPR = KD / 8;
  static constexpr int LPR = (CPR % 64 == 0) ? 64 : (CPR % 32 == 0) ? 32 : (CPR % 16 == 0) ? 16 : (CPR % 8 == 0) ? 8 : 4;
  static constexpr int RPP = 64 / LPR;
  static constexpr int CPL = CPR / LPR;
  static_assert(CPR % LPR == 0, "row length must be a multiple of 8*LPR words");
};

// A block of NP row passes: 16-byte loads of weights (KD = 16-bit words of codes per row) and,
// for FP8 rows (WF 1), each row's scale; for MXFP4 rows (WF 2), each 16-byte chunk's block scale
template <int KD, int NP, int WF = 0>
struct WBuf {
  u4 w[NP][Geo<KD>::CPL];
  float s[WF == 2 ? NP * Geo<KD>::CPL : WF == 1 ? NP : 1];
};

template <int KD, int NP>
__device__ __forceinline__ int block_rows() { return NP * NWAVE * Geo<KD>::RPP; }

// RowPtr(r) -> const uint16_t* start of row r (only called for r < nrows); an FP8 row's scale is the
// float right after its KD words of codes; an MXFP4 row's block scales are the bytes right after
// its codes, one per 16-byte chunk (chunk c of the row: byte c)
template <int KD, int NP, int WF = 0, class RowPtr>
__device__ __forceinline__ void load_block(WBuf<KD, NP, WF>& b, int blk, int nrows, RowPtr rowptr) {
  using G = Geo<KD>;
  const int tx = tid(), lane = tx & 63, wave = __builtin_amdgcn_readfirstlane(tx >> 6);
  const int rip = lane / G::LPR, lir = lane % G::LPR;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int r = ((blk * NP + i) * NWAVE + wave) * G::RPP + rip;
    if (r < nrows) {
      const uint16_t* src = rowptr(r) + 8 * lir;
#pragma unroll
      for (int j = 0; j < G::CPL; ++j) b.w[i][j] = ldw(src + 8 * G::LPR * j);
      if constexpr (WF == 1) b.s[i] = *reinterpret_cast<const float*>(rowptr(r) + KD);
      if constexpr (WF == 2) {
        const uint8_t* sb = reinterpret_cast<const uint8_t*>(rowptr(r) + KD) + lir;
#pragma unroll
        for (int j = 0; j < G::CPL; ++j) b.s[i * G::CPL + j] = e8m0(sb[G::LPR * j]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < G::CPL; ++j) b.w[i][j] = u4{0u, 0u, 0u, 0u};
      if constexpr (WF == 1) b.s[i] = 0.f;
      if constexpr (WF == 2) {
#pragma unroll
        for (int j = 0; j < G::CPL; ++j) b.s[i * G::CPL + j] = 0.f;
      }
    }
  }
}

// ActOf(r, t) -> const float* LDS activations (KD floats) for row r, token t
// Emit(r, t, value) is called on the lane with lir == 0 of each row (value = full dot product)
// (FP8 rows: 16 inputs per 16-byte load, and each row's sum times its scale; MXFP4 rows: 32 inputs
// per load, each chunk's sum times its block scale)
template <int KD, int NP, int TB, int WF = 0, class ActOf, class Emit>
__device__ __forceinline__ void compute_block(const WBuf<KD, NP, WF>& b, int blk, int nrows, int ntok,
                                              ActOf act_of, Emit emit) {
  constexpr int EPC = WF == 2 ? 32 : WF == 1 ? 16 : 8;
  using G = Geo<KD>;
  const int tx = tid(), lane = tx & 63, wave = __builtin_amdgcn_readfirstlane(tx >> 6);
  const int rip = lane / G::LPR, lir = lane % G::LPR;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int r = ((blk * NP + i) * NWAVE + wave) * G::RPP + rip;
    const int rr = r < nrows ? r : 0;
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      if (t < ntok) {
        const float* a = act_of(rr, t) + EPC * lir;
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < G::CPL; ++j) {
          const f4* ap = reinterpret_cast<const f4*>(a + EPC * G::LPR * j);
          if constexpr (WF == 2) {
            const u4 w = b.w[i][j];
            const float sc = b.s[i * G::CPL + j];
            acc = dot8f(dec8e2m1(w.x, sc), ap[0], ap[1], acc);
            acc = dot8f(dec8e2m1(w.y, sc), ap[2], ap[3], acc);
            acc = dot8f(dec8e2m1(w.z, sc), ap[4], ap[5], acc);
            acc = dot8f(dec8e2m1(w.w, sc), ap[6], ap[7], acc);
          } else if constexpr (WF == 1) acc = dot16e4m3(b.w[i][j], ap[0], ap[1], ap[2], ap[3], acc);
          else acc = dot8(b.w[i][j], ap[0], ap[1], acc);
        }
        acc = wsum<G::LPR>(acc);
        if constexpr (WF == 1) acc *= b.s[i];
        if (lir == 0 && r < nrows) emit(r, t, acc);
      }
    }
  }
}

// compute_block for activations that do not depend on the row (every GEMV whose rows share one
// input vector per token): each 16-byte activation read from LDS serves all NP passes of the block,
// so a batch of TB tokens reads LDS NP times less. Per row, the products are summed in the same
// order as compute_block.
//
// TG = 2 (tokens that share every row: the batch in the QKV and router GEMVs of the vector-ALU form,
// the tokens of a union slot in bf16 expert items): tokens are taken in pairs, so that each weight
// is unpacked from bf16 once per pair (such GEMVs are bound by vector-ALU issue at several tokens). A pair is computed whole once its first token is in range (act_of must return readable
// LDS for every t < TB); the second token's result is emitted only if it is in range. Same per-row
// order of products.
//
// TG = 4 (MXFP4 rows that every token of the batch multiplies: lm_head, the O projection): groups of
// up to 4 tokens share each conversion, under the same rule; bf16 and FP8 rows take the tokens one
// at a time there (TG_ROWS below).
template <int KD, int NP, int TB, int TG = 1, int WF = 0, class ActOf, class Emit>
__device__ __forceinline__ void compute_block_shared(const WBuf<KD, NP, WF>& b, int blk, int nrows, int ntok,
                                                     ActOf act_of, Emit emit) {
  using G = Geo<KD>;
  constexpr int EPC = WF == 2 ? 32 : WF == 1 ? 16 : 8;
  const int tx = tid(), lane = tx & 63, wave = __builtin_amdgcn_readfirstlane(tx >> 6);
  const int rip = lane / G::LPR, lir = lane % G::LPR;
  if constexpr (TG == 2) {
    static_assert(TB % 2 == 0, "");
#pragma unroll
    for (int t0 = 0; t0 < TB; t0 += 2) {
      if (t0 < ntok) {
        const float* pa = act_of(0, t0) + EPC * lir;
        const float* pb = act_of(0, t0 + 1) + EPC * lir;
        float acc0[NP], acc1[NP];
#pragma unroll
        for (int i = 0; i < NP; ++i) { acc0[i] = 0.f; acc1[i] = 0.f; }
#pragma unroll
        for (int j = 0; j < G::CPL; ++j) {
          const f4* qa = reinterpret_cast<const f4*>(pa + EPC * G::LPR * j);
          const f4* qb = reinterpret_cast<const f4*>(pb + EPC * G::LPR * j);
          if constexpr (WF == 2) {
            // 32 codes per load, a dword (8 codes) at a time: the pair's two tokens share each
            // conversion
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const f4 a0 = qa[2 * k], a1 = qa[2 * k + 1], c0 = qb[2 * k], c1 = qb[2 * k + 1];
#pragma unroll
              for (int i = 0; i < NP; ++i) {
                const u4 w = b.w[i][j];
                const f8v d = dec8e2m1(k == 0 ? w.x : k == 1 ? w.y : k == 2 ? w.z : w.w, b.s[i * G::CPL + j]);
                acc0[i] = dot8f(d, a0, a1, acc0[i]);
                acc1[i] = dot8f(d, c0, c1, acc1[i]);
              }
            }
            continue;
          }
          if constexpr (WF == 1) {
            // 16 codes per load: the pair's two tokens share each conversion
            const f4 a[4] = {qa[0], qa[1], qa[2], qa[3]}, c[4] = {qb[0], qb[1], qb[2], qb[3]};
#pragma unroll
            for (int i = 0; i < NP; ++i) {
              const u4 w = b.w[i][j];
              const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
              float x = acc0[i], y = acc1[i];
#pragma unroll
              for (int k = 0; k < 4; ++k) {
                const f2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(wd[k], false), hi = __builtin_amdgcn_cvt_pk_f32_fp8(wd[k], true);
                x = __builtin_fmaf(lo.x, a[k].x, x); y = __builtin_fmaf(lo.x, c[k].x, y);
                x = __builtin_fmaf(lo.y, a[k].y, x); y = __builtin_fmaf(lo.y, c[k].y, y);
                x = __builtin_fmaf(hi.x, a[k].z, x); y = __builtin_fmaf(hi.x, c[k].z, y);
                x = __builtin_fmaf(hi.y, a[k].w, x); y = __builtin_fmaf(hi.y, c[k].w, y);
              }
              acc0[i] = x; acc1[i] = y;
            }
            continue;
          }
          const f4 a0 = qa[0], a1 = qa[1], b0 = qb[0], b1 = qb[1];
#pragma unroll
          for (int i = 0; i < NP; ++i) {
            const u4 w = b.w[i][j];
            const float wf[8] = {bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y),
                                 bf_lo(w.z), bf_hi(w.z), bf_lo(w.w), bf_hi(w.w)};
            float x = acc0[i], y = acc1[i];
            x = __builtin_fmaf(wf[0], a0.x, x); y = __builtin_fmaf(wf[0], b0.x, y);
            x = __builtin_fmaf(wf[1], a0.y, x); y = __builtin_fmaf(wf[1], b0.y, y);
            x = __builtin_fmaf(wf[2], a0.z, x); y = __builtin_fmaf(wf[2], b0.z, y);
            x = __builtin_fmaf(wf[3], a0.w, x); y = __builtin_fmaf(wf[3], b0.w, y);
            x = __builtin_fmaf(wf[4], a1.x, x); y = __builtin_fmaf(wf[4], b1.x, y);
            x = __builtin_fmaf(wf[5], a1.y, x); y = __builtin_fmaf(wf[5], b1.y, y);
            x = __builtin_fmaf(wf[6], a1.z, x); y = __builtin_fmaf(wf[6], b1.z, y);
            x = __builtin_fmaf(wf[7], a1.w, x); y = __builtin_fmaf(wf[7], b1.w, y);
            acc0[i] = x; acc1[i] = y;
          }
        }
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          const int r = ((blk * NP + i) * NWAVE + wave) * G::RPP + rip;
          float v0 = wsum<G::LPR>(acc0[i]), v1 = wsum<G::LPR>(acc1[i]);
          if constexpr (WF == 1) { v0 *= b.s[i]; v1 *= b.s[i]; }
          if (lir == 0 && r < nrows) {
            emit(r, t0, v0);
            if (t0 + 1 < ntok) emit(r, t0 + 1, v1);
          }
        }
      }
    }
    return;
  }
  if constexpr (WF == 2 && TG == 4) {
    // MXFP4, tokens in groups of up to 4 (every token of the batch multiplies every row: lm_head, the
    // O projection): each dword's conversions serve the group (a pass's 8 decoded weights meet each
    // token's 8 activations). A group is computed whole once its first token is in range (act_of
    // must return readable LDS for every t < TB); results are emitted for tokens in range only
    constexpr int TQ = TB < 4 ? TB : 4;
#pragma unroll
    for (int t0 = 0; t0 < TB; t0 += TQ) {
      if (t0 < ntok) {
        float acc[TQ][NP];
#pragma unroll
        for (int t = 0; t < TQ; ++t)
#pragma unroll
          for (int i = 0; i < NP; ++i) acc[t][i] = 0.f;
#pragma unroll
        for (int j = 0; j < G::CPL; ++j) {
          // (the chunk's 4 dwords in a loop that is not unrolled: unrolled, the compiler hoisted
          // every conversion and activation read of the chunk ahead of the products)
          u4 wv[NP];
          float sc[NP];
#pragma unroll
          for (int i = 0; i < NP; ++i) { wv[i] = b.w[i][j]; sc[i] = b.s[i * G::CPL + j]; }
          const f4* ab[TQ];
#pragma unroll
          for (int t = 0; t < TQ; ++t) ab[t] = reinterpret_cast<const f4*>(act_of(0, t0 + t) + EPC * lir + EPC * G::LPR * j);
#pragma unroll 1
          for (int k = 0; k < 4; ++k) {
            f4 a0[TQ], a1[TQ];
#pragma unroll
            for (int t = 0; t < TQ; ++t) {
              a0[t] = ab[t][2 * k];
              a1[t] = ab[t][2 * k + 1];
            }
#pragma unroll
            for (int i = 0; i < NP; ++i) {
              const f8v d = dec8e2m1(wv[i].x, sc[i]);
#pragma unroll
              for (int t = 0; t < TQ; ++t) acc[t][i] = dot8f(d, a0[t], a1[t], acc[t][i]);
              wv[i] = u4{wv[i].y, wv[i].z, wv[i].w, 0u};
            }
          }
        }
#pragma unroll
        for (int t = 0; t < TQ; ++t) {
#pragma unroll
          for (int i = 0; i < NP; ++i) {
            const int r = ((blk * NP + i) * NWAVE + wave) * G::RPP + rip;
            const float v = wsum<G::LPR>(acc[t][i]);
            if (lir == 0 && r < nrows && t0 + t < ntok) emit(r, t0 + t, v);
          }
        }
      }
    }
    return;
  }
  if constexpr (WF == 2) {
    // MXFP4, one token at a time (items whose rows few tokens share: expert gate/up and down); the
    // chunk's dwords in a loop that is not unrolled, as above
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      if (t < ntok) {
        const float* a = act_of(0, t) + EPC * lir;
        float acc[NP];
#pragma unroll
        for (int i = 0; i < NP; ++i) acc[i] = 0.f;
#pragma unroll
        for (int j = 0; j < G::CPL; ++j) {
          const f4* ap = reinterpret_cast<const f4*>(a + EPC * G::LPR * j);
          u4 wv[NP];
          float sc[NP];
#pragma unroll
          for (int i = 0; i < NP; ++i) { wv[i] = b.w[i][j]; sc[i] = b.s[i * G::CPL + j]; }
#pragma unroll 1
          for (int k = 0; k < 4; ++k) {
            const f4 a0 = ap[2 * k], a1 = ap[2 * k + 1];
#pragma unroll
            for (int i = 0; i < NP; ++i) {
              acc[i] = dot8f(dec8e2m1(wv[i].x, sc[i]), a0, a1, acc[i]);
              wv[i] = u4{wv[i].y, wv[i].z, wv[i].w, 0u};
            }
          }
        }
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          const int r = ((blk * NP + i) * NWAVE + wave) * G::RPP + rip;
          const float v = wsum<G::LPR>(acc[i]);
          if (lir == 0 && r < nrows) emit(r, t, v);
        }
      }
    }
    return;
  }
#pragma unroll
  for (int t = 0; t < TB; ++t) {
    if (t < ntok) {
      const float* a = act_of(0, t) + EPC * lir;
      float acc[NP];
#pragma unroll
      for (int i = 0; i < NP; ++i) acc[i] = 0.f;
#pragma unroll
      for (int j = 0; j < G::CPL; ++j) {
        const f4* ap = reinterpret_cast<const f4*>(a + EPC * G::LPR * j);
        if constexpr (WF == 1) {
          const f4 a0 = ap[0], a1 = ap[1], a2 = ap[2], a3 = ap[3];
#pragma unroll
          for (int i = 0; i < NP; ++i) acc[i] = dot16e4m3(b.w[i][j], a0, a1, a2, a3, acc[i]);
        } else {
          const f4 a0 = ap[0], a1 = ap[1];
#pragma unroll
          for (int i = 0; i < NP; ++i) acc[i] = dot8(b.w[i][j], a0, a1, acc[i]);
        }
      }
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int r = ((blk * NP + i) * NWAVE + wave) * G::RPP + rip;
        float v = wsum<G::LPR>(acc[i]);
        if constexpr (WF == 1) v *= b.s[i];
        if (lir == 0 && r < nrows) emit(r, t, v);
      }
    }
  }
}

// token grouping of a GEMV whose rows every token of the step multiplies, besides QKV and router
template <class S>
constexpr int TG_ROWS = S::WF == 2 ? 4 : 1;

// Stream `nrows` rows; block 0 may already be loaded into A (prefetched before a dependency wait).
// The activations are shared by all rows (ActOf ignores its row argument).
template <int KD, int NP, int TB, int TG = 1, int WF = 0, class RowPtr, class ActOf, class Emit>
__device__ __forceinline__ void gemv_stream(WBuf<KD, NP, WF>& A, bool a_loaded, int nrows, int ntok,
                                            RowPtr rowptr, ActOf act_of, Emit emit) {
  const int nblk = (nrows + block_rows<KD, NP>() - 1) / block_rows<KD, NP>();
  WBuf<KD, NP, WF> B;
  if (!a_loaded) load_block<KD, NP, WF>(A, 0, nrows, rowptr);
  for (int blk = 0; blk < nblk; blk += 2) {
    if (blk + 1 < nblk) load_block<KD, NP, WF>(B, blk + 1, nrows, rowptr);
    compute_block_shared<KD, NP, TB, TG, WF>(A, blk, nrows, ntok, act_of, emit);
    if (blk + 1 < nblk) {
      if (blk + 2 < nblk) load_block<KD, NP, WF>(A, blk + 2, nrows, rowptr);
      compute_block_shared<KD, NP, TB, TG, WF>(B, blk + 1, nrows, ntok, act_of, emit);
    }
  }
}

// ------------------------------------------------------------------------------ matrix-core rows
//
// Rows of a matrix times the step's tokens on the matrix cores (batch > 1; P3 "Key Technologies and
// Architecture": the dense contractions on the tensor cores), with v_mfma_f32_16x16x32_bf16.
//
// A operand: a row block is 16 rows; each wave covers a quarter of the inputs. Lane l holds row
// l % 16 and, per load, EPL consecutive inputs of it: lane group q = l / 16 the q-th EPL inputs of
// the load's span of 4 EPL. A product takes 8 of each lane's inputs (the k index of the product
// is a permutation of the inputs, the same for both operands). bf16 rows: 8 inputs per 16-byte
// load. FP8 rows: 16 codes per 16-byte load, converted to bf16 (exact: E4M3 values have 4
// significant bits), the row's scale applied to the finished sum. MXFP4 rows: 16 codes per 8-byte
// load, converted to bf16 with their block's scale (exact: a 2-bit significand times a power of two).
//
// B operand: the activations stay fp32 in LDS; each lane splits the 8 it feeds into three bf16
// parts, hi = bf16(x), lo = bf16(x - hi), lo2 = bf16(x - hi - lo): each difference is exact and x is
// their exact sum, so the products are exact and a row carries the error of an fp32 sum, as the
// vector-ALU form does. Two products per 8 inputs in one accumulator chain: column c of the first is
// token c % 8's hi part (c < 8) or lo part (c >= 8), of the second its lo2 part (c < 8) or zero.
// The four waves' 16 x 16 sums are added in LDS in wave order, then column t + column t + 8.

typedef __bf16 bf8v __attribute__((ext_vector_type(8)));
typedef __bf16 bf2v __attribute__((ext_vector_type(2)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

template <class S>
struct MRows {
  static constexpr int WF = S::WF;
  static constexpr int EPL = WF == 0 ? 8 : 16;     // inputs of a lane per load
  static constexpr int SPAN = 4 * EPL;             // inputs of a wave per load
  static constexpr int NL = S::H / NWAVE / SPAN;   // loads per wave and row block
  static constexpr int AS = S::H + 4;         // LDS row stride of the staged activations (floats;
                                              // the pad puts the 8 tokens' reads in distinct banks)
  static constexpr int RED = MAXB * AS;       // then [NWAVE][16][16] float partial sums
  static constexpr int SC = RED + NWAVE * 256;   // then [16] row scales (FP8)
  static constexpr int END = SC + 16;
  static_assert((S::H / NWAVE) % SPAN == 0 && AS % 4 == 0, "");
  typedef typename std::conditional<WF == 2, u2, u4>::type LT;
  LT a[NL];
  float s[WF == 2 ? NL : 1];                  // MXFP4: each load's block scale; FP8: the row's scale
};

// A operand of row block rb (rows rb*16 ..); rows at or past nrows are zeros
template <class S, class RowPtr>
__device__ __forceinline__ void mrows_load(MRows<S>& A, int rb, int nrows, RowPtr rowptr) {
  using M = MRows<S>;
  const int lane = tid() & 63, wave = __builtin_amdgcn_readfirstlane(tid() >> 6);
  const int r = rb * 16 + (lane & 15);
  const int e0 = S::H / NWAVE * wave + M::EPL * (lane >> 4);     // first input of the lane's load 0
  if (r < nrows) {
    const uint16_t* row = rowptr(r);
    const uint8_t* rb8 = reinterpret_cast<const uint8_t*>(row);
#pragma unroll
    for (int j = 0; j < M::NL; ++j) {
      const int e = e0 + M::SPAN * j;
      if constexpr (M::WF == 0) A.a[j] = ldw(row + e);
      if constexpr (M::WF == 1) A.a[j] = ldw(rb8 + e);
      if constexpr (M::WF == 2) {
        A.a[j] = __builtin_nontemporal_load(reinterpret_cast<const u2*>(rb8 + e / 2));
        A.s[j] = e8m0(rb8[S::H / 2 + e / 32]);
      }
    }
    if constexpr (M::WF == 1) A.s[0] = *reinterpret_cast<const float*>(rb8 + S::H);
  } else {
#pragma unroll
    for (int j = 0; j < M::NL; ++j) {
      if constexpr (M::WF == 2) { A.a[j] = u2{0u, 0u}; A.s[j] = 0.f; }
      else A.a[j] = u4{0u, 0u, 0u, 0u};
    }
    if constexpr (M::WF == 1) A.s[0] = 0.f;
  }
}

// two bf16 of a float pair, packed (round to nearest even)
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{a, b}, bf2v));
}

// Products of row block rb with the staged tokens (act: [MAXB][AS] fp32); emit(r, t, value) for rows
// r < nrows and tokens t < ntok, on threads 0..127 (thread 8 i + t: row rb*16 + i, token t). Ends
// with a barrier.
template <class S, class Emit>
__device__ __forceinline__ void mrows_compute(const MRows<S>& A, int rb, int nrows, int ntok, const float* act,
                                              float* red, Emit emit) {
  using M = MRows<S>;
  const int tx = tid(), lane = tx & 63, wave = __builtin_amdgcn_readfirstlane(tx >> 6);
  const int col = lane & 15, kq = lane >> 4;
  const bool first = col < 8;
  const float* xs = act + (col & 7) * M::AS + S::H / NWAVE * wave + M::EPL * kq;
  f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < M::NL; ++j) {
    u4 af[M::EPL / 8];                 // the lane's inputs as bf16, 8 per product
    if constexpr (M::WF == 0) af[0] = A.a[j];
    if constexpr (M::WF == 1) {
      const uint32_t w[4] = {A.a[j].x, A.a[j].y, A.a[j].z, A.a[j].w};
      uint32_t d[8];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        d[2 * m] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[m], 1.0f, false));
        d[2 * m + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[m], 1.0f, true));
      }
      af[0] = u4{d[0], d[1], d[2], d[3]};
      af[1] = u4{d[4], d[5], d[6], d[7]};
    }
    if constexpr (M::WF == 2) {
      const uint32_t w[2] = {A.a[j].x, A.a[j].y};
      const float sc = A.s[j];
      uint32_t d[8];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        d[4 * m] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[m], sc, 0));
        d[4 * m + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[m], sc, 1));
        d[4 * m + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[m], sc, 2));
        d[4 * m + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[m], sc, 3));
      }
      af[0] = u4{d[0], d[1], d[2], d[3]};
      af[1] = u4{d[4], d[5], d[6], d[7]};
    }
#pragma unroll
    for (int m = 0; m < M::EPL / 8; ++m) {
      const float* xp = xs + M::SPAN * j + 8 * m;
      const f4 x0 = *reinterpret_cast<const f4*>(xp), x1 = *reinterpret_cast<const f4*>(xp + 4);
      const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      uint32_t b1[4], b2[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t h = pk_bf16(x[2 * q], x[2 * q + 1]);
        const float r0 = x[2 * q] - bf_lo(h), r1 = x[2 * q + 1] - bf_hi(h);
        const uint32_t l = pk_bf16(r0, r1);
        const uint32_t l2 = pk_bf16(r0 - bf_lo(l), r1 - bf_hi(l));
        b1[q] = first ? h : l;
        b2[q] = first ? l2 : 0u;
      }
      const bf8v a = __builtin_bit_cast(bf8v, af[m]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf8v, u4{b1[0], b1[1], b1[2], b1[3]}), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf8v, u4{b2[0], b2[1], b2[2], b2[3]}), acc, 0, 0, 0);
    }
  }
  // (the product's lane holds column col, rows 4 kq .. 4 kq + 3)
#pragma unroll
  for (int i = 0; i < 4; ++i) red[(wave * 16 + 4 * kq + i) * 16 + col] = acc[i];
  if constexpr (M::WF == 1)
    if (wave == 0 && kq == 0) red[M::SC - M::RED + col] = A.s[0];     // row col's scale
  __syncthreads();
  if (tx < 128) {
    const int i = tx >> 3, t = tx & 7;
    float a0 = red[i * 16 + t], a1 = red[i * 16 + 8 + t];
#pragma unroll
    for (int w = 1; w < NWAVE; ++w) {
      a0 += red[(w * 16 + i) * 16 + t];
      a1 += red[(w * 16 + i) * 16 + 8 + t];
    }
    float v = a0 + a1;
    if constexpr (M::WF == 1) v *= red[M::SC - M::RED + i];
    const int r = rb * 16 + i;
    if (r < nrows && t < ntok) emit(r, t, v);
  }
  __syncthreads();
}

// Every row block of nrows rows, the next block's loads in flight while one is multiplied (block 0
// may already be loaded into A, before a dependency wait)
template <class S, class RowPtr, class Emit>
__device__ __forceinline__ void mrows_stream(MRows<S>& A, bool a_loaded, int nrows, int ntok, RowPtr rowptr,
                                             const float* act, float* red, Emit emit) {
  const int nblk = (nrows + 15) / 16;
  MRows<S> A2;
  if (!a_loaded) mrows_load<S>(A, 0, nrows, rowptr);
  for (int rb = 0; rb < nblk; rb += 2) {
    if (rb + 1 < nblk) mrows_load<S>(A2, rb + 1, nrows, rowptr);
    mrows_compute<S>(A, rb, nrows, ntok, act, red, emit);
    if (rb + 1 < nblk) {
      if (rb + 2 < nblk) mrows_load<S>(A, rb + 2, nrows, rowptr);
      mrows_compute<S>(A2, rb + 1, nrows, ntok, act, red, emit);
    }
  }
}

// ------------------------------------------------------------------------------ norm staging

// act[t][H] = RMSNorm(x_l[b_t]) * gain for the listed tokens (P1: one shared normed input per
// layer). x_0 is the token's embedding row; x_l (l >= 1) comes from the previous layer's OUT
// tasks. One wave per token: each lane sums H/64 squares, then a wave tree.
// AS: the row stride of act (floats; the matrix-core form pads its rows).
template <class S, int AS = S::H>
__device__ __forceinline__ void stage_norm(CParams& p, int l, const int* toks, int ntok, const uint16_t* gain,
                           float* act, int task) {
  constexpr int H = S::H;
  constexpr int G4 = H / 256;            // groups of 4 consecutive floats per lane
  static_assert(H % 256 == 0, "");
  const int tx = tid(), lane = tx & 63, wave = __builtin_amdgcn_readfirstlane(tx >> 6);
  uint2 gw[G4];                          // the gain, requested together with the activations
  if (wave < ntok) {
#pragma unroll
    for (int k = 0; k < G4; ++k) gw[k] = *reinterpret_cast<const uint2*>(gain + 4 * lane + 256 * k);
  }
  for (int t = wave; t < ntok; t += NWAVE) {
    const int b = toks[t];
    float v[4 * G4];
    if (l == 0) {
      int tok = cst(p.tokens)[b];
      if (tok < 0 || tok >= p.V) {
        if (lane == 0) raise_error(p, DEV_BAD_TOKEN, task, -1, 0, (uint32_t)tok, (uint32_t)b);
        tok = 0;
      }
      const uint16_t* row = p.embed + (size_t)tok * H;
#pragma unroll
      for (int k = 0; k < G4; ++k) {
        const uint2 w = *reinterpret_cast<const uint2*>(row + 4 * lane + 256 * k);
        v[4 * k + 0] = bf_lo(w.x); v[4 * k + 1] = bf_hi(w.x);
        v[4 * k + 2] = bf_lo(w.y); v[4 * k + 3] = bf_hi(w.y);
      }
    } else {
      const __amdgpu_buffer_rsrc_t X = rsrc(p.x + ((size_t)l * MAXB + b) * H);
#pragma unroll
      for (int k = 0; k < G4; ++k) {
        const f4 a = ldc4(X, 4u * (4 * lane + 256 * k));
        v[4 * k + 0] = a.x; v[4 * k + 1] = a.y; v[4 * k + 2] = a.z; v[4 * k + 3] = a.w;
      }
    }
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < 4 * G4; ++k) ss = __builtin_fmaf(v[k], v[k], ss);
    ss = wsum<64>(ss);
    const float inv = 1.0f / sqrtf(ss / (float)H + p.eps);
#pragma unroll
    for (int k = 0; k < G4; ++k) {
      const float gg[4] = {bf_lo(gw[k].x), bf_hi(gw[k].x), bf_lo(gw[k].y), bf_hi(gw[k].y)};
      f4 o;
      o.x = (v[4 * k + 0] * inv) * gg[0];
      o.y = (v[4 * k + 1] * inv) * gg[1];
      o.z = (v[4 * k + 2] * inv) * gg[2];
      o.w = (v[4 * k + 3] * inv) * gg[3];
      *reinterpret_cast<f4*>(act + (size_t)t * AS + 4 * lane + 256 * k) = o;
    }
  }
  __syncthreads();
}

// ------------------------------------------------------------------------------ ops

struct TaskHdr {
  int id, op, layer, a0, a1, a2, a3, a4, a5, w0, t0, w1, t1, sig, sig2;
};

// Fields of task `ti` (uniform: the descriptor is read with scalar loads).
__device__ __forceinline__ TaskHdr read_task(CParams& p, int ti) {
  ti = __builtin_amdgcn_readfirstlane(ti);
  const __attribute__((address_space(4))) int32_t* d = cst(p.tasks) + (size_t)ti * DESC_WORDS;
  TaskHdr T;
  T.id = ti;
  T.op = d[D_OP]; T.layer = d[D_LAYER];
  T.a0 = d[D_A0]; T.a1 = d[D_A1]; T.a2 = d[D_A2]; T.a3 = d[D_A3]; T.a4 = d[D_A4]; T.a5 = d[D_A5];
  T.w0 = d[D_W0]; T.t0 = d[D_T0]; T.w1 = d[D_W1]; T.t1 = d[D_T1];
  T.sig = d[D_SIG]; T.sig2 = d[D_SIG2];
  return T;
}

template <class S, int TB>
__device__ __forceinline__ float* rope_tab();

// The cache rows of this step's tokens, published by the QKV task that produced them (kernel
// instance for batches whose rows are consecutive positions of one sequence: chunked prefill and
// mixed prefill/decode batches). Tile [row0, row0 + nrows) of the K rows (one whole head, so that
// RoPE's rotate-half partners are in the tile) or of the V rows: every row's fp32 outputs, already
// stored and drained by this workgroup, are read back, K rotated by RoPE at the row's position
// (R3 of the oracle's readings, as the attention forms the new key), both rounded to bf16 and
// written at the row's slot with write-through stores (R6). The caller drains before it signals, so
// an attention task that has seen the QKV counter reads every row's key from the cache.
template <class S, int TB>
__device__ __forceinline__ bool publish_kv(CParams& p, int l, int row0, int nrows, int task) {
  constexpr int D = S::D, HQ = S::HQ, HKV = S::HKV;
  const bool is_k = row0 < (HQ + HKV) * D;
  const int base = is_k ? HQ * D : (HQ + HKV) * D;
  const int g = (row0 - base) / D, dlo = (row0 - base) % D;
  if ((is_k && (dlo != 0 || nrows != D)) || (!is_k && (nrows % 8 != 0 || dlo % 8 != 0 || dlo + nrows > D))) {
    if (tid() == 0) raise_error(p, DEV_BAD_OP, task, -1, (uint32_t)row0, (uint32_t)nrows, 0);
    return false;
  }
  const auto& Lp = cst(p.layers)[l];
  uint16_t* cache = is_k ? Lp.k_cache : Lp.v_cache;
  const int nch = nrows / 8;                       // 8 dims (one 16-byte store) per item
  uint32_t bad = 0, bad_a = 0, bad_b = 0;          // the first refused item (reported after the loop)
  for (int i = tid(); i < p.B * nch; i += NT) {
    const int b = i / nch, d0 = dlo + 8 * (i % nch);
    const int pos = cst(p.positions)[b];
    if (pos < 0 || pos >= p.max_pages * PAGE) {
      if (!bad) { bad = DEV_BAD_POS; bad_a = (uint32_t)pos; bad_b = (uint32_t)b; }
      continue;
    }
    const int page = cst(p.block_tables)[(size_t)b * p.max_pages + pos / PAGE];
    if (page < 0 || page >= p.num_pages) {
      if (!bad) { bad = DEV_BAD_PAGE; bad_a = (uint32_t)page; bad_b = (uint32_t)(pos / PAGE); }
      continue;
    }
    const __amdgpu_buffer_rsrc_t Q = rsrc(p.qkv + ((size_t)l * MAXB + b) * S::QKVR);
    const uint32_t src = (uint32_t)(base + g * D + d0);
    const f4 x0 = ldc4(Q, 4u * src), x1 = ldc4(Q, 4u * (src + 4));
    float r[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    if (is_k) {
      const int pd0 = d0 < D / 2 ? d0 + D / 2 : d0 - D / 2;
      const uint32_t ps = (uint32_t)(base + g * D + pd0);
      const f4 y0 = ldc4(Q, 4u * ps), y1 = ldc4(Q, 4u * (ps + 4));
      const float y[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
      const float* cs = rope_tab<S, TB>() + b * D;   // [D/2] cos, [D/2] sin at pos
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int j = (d0 + m) % (D / 2);
        const float c = cs[j], sn = cs[D / 2 + j];
        r[m] = d0 < D / 2 ? r[m] * c - y[m] * sn : r[m] * c + y[m] * sn;
      }
    }
    u4 w;
    w.x = f2bf(r[0]) | (f2bf(r[1]) << 16); w.y = f2bf(r[2]) | (f2bf(r[3]) << 16);
    w.z = f2bf(r[4]) | (f2bf(r[5]) << 16); w.w = f2bf(r[6]) | (f2bf(r[7]) << 16);
    const __amdgpu_buffer_rsrc_t C = rsrc(cache + ((size_t)page * HKV + g) * PAGE * D);
    __builtin_amdgcn_raw_buffer_store_b128(w, C, (uint32_t)(((pos % PAGE) * D + d0) * 2), 0, SC1);
  }
  if (bad)
    raise_error(p, bad, task, -1, bad == DEV_BAD_POS ? (uint32_t)p.max_pages : (uint32_t)p.num_pages, bad_a, bad_b);
  return __syncthreads_or(bad != 0) == 0;
}

// dst[0, n) = the n floats at byte offset off of R (n a multiple of 4, at most NMAX): every load of
// the thread is issued before its first LDS write, so the staging costs one round trip
template <int NMAX>
__device__ __forceinline__ void stage_f4(float* dst, __amdgpu_buffer_rsrc_t R, uint32_t off, int n) {
  constexpr int NI = (NMAX + 4 * NT - 1) / (4 * NT);
  const int tx = tid();
  f4 v[NI];
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    const int i = (u * NT + tx) * 4;
    v[u] = i < n ? ldc4(R, off + 4u * i) : f4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    const int i = (u * NT + tx) * 4;
    if (i < n) *reinterpret_cast<f4*>(dst + i) = v[u];
  }
}

// QKV rows (any contiguous range inside one KV group's q, k or v rows).
template <class S, int TB, int VAR>
__device__ __forceinline__ bool op_qkv(int task) {
  CParams& p = P();
  Ctl& ctl = ctl_s;
  float* sm = smem;
  const TaskHdr T = read_task(p, task);
  // a whole 16-row tile in flight before the wait (FP8 rows: 4 passes too, the register budget of the
  // batch form's token pairs)
  constexpr int H = S::H, KW = S::kw(H), NP = (Geo<KW>::CPL >= 4 || S::WF) ? 4 : 8;
  const auto& Lp = cst(p.layers)[T.layer];
  const int row0 = T.a0, nrows = T.a1;
  auto rowptr = [&](int r) { return Lp.w_qkv + (size_t)(row0 + r) * S::rw(H); };
  const bool pre = !(p.flags & 2);
  const __amdgpu_buffer_rsrc_t Q = rsrc(p.qkv + (size_t)T.layer * MAXB * S::QKVR);
  auto emit = [&](int r, int t, float v) { stc(Q, 4u * (t * S::QKVR + row0 + r), v); };
  if constexpr (TB > 1) {                        // several tokens: the matrix cores
    MRows<S> A;
    if (pre) mrows_load<S>(A, 0, nrows, rowptr);
    if (!wait_ge(p, ctl, T.w0, (uint32_t)T.t0, T.id)) return false;
    if (tid() < MAXB) ctl.toks[tid()] = tid();
    __syncthreads();
    stage_norm<S, MRows<S>::AS>(p, T.layer, ctl.toks, p.B, Lp.attn_norm, sm, T.id);
    MARK(0);
    mrows_stream<S>(A, pre, nrows, p.B, rowptr, sm, sm + MRows<S>::RED, emit);
  } else {
    WBuf<KW, NP, S::WF> A;
    if (pre) load_block<KW, NP, S::WF>(A, 0, nrows, rowptr);
    if (!wait_ge(p, ctl, T.w0, (uint32_t)T.t0, T.id)) return false;
    if (tid() < MAXB) ctl.toks[tid()] = tid();
    __syncthreads();
    stage_norm<S>(p, T.layer, ctl.toks, p.B, Lp.attn_norm, sm, T.id);
    MARK(0);
    gemv_stream<KW, NP, TB, (TB > 1 ? 2 : 1), S::WF>(A, pre, nrows, p.B, rowptr,
        [&](int r, int t) { return sm + (size_t)t * H; }, emit);
  }
  MARK(1);
  drain_t(p);
  if constexpr (VAR == 2) {
    if (row0 >= S::HQ * S::D) {          // a K or V tile: the rows' cache entries, before the signal
      __syncthreads();                   // every thread's stores of the tile have landed
      const bool ok = publish_kv<S, TB>(p, T.layer, row0, nrows, T.id);   // (uniform)
      drain();
      if (!ok) return false;
    }
  }
  MARK(2);
  signal(p, ctl, T.sig, false);
  return true;
}

// Top-k of token b's router logits on one wave (R7 of the oracle's readings: ties go to the lower
// expert index), returned in ascending expert order with the selection as a 128-bit mask. Every
// consumer of a routing decision runs this same selection on the same logits, so they agree exactly.
template <class S>
__device__ __forceinline__ void topk_select(CParams& p, int l, int b, int lane, bool emit, int (&widx)[S::K],
                                            float (&wval)[S::K], unsigned long long& m0, unsigned long long& m1) {
  constexpr int E = S::E, K = S::K, EPL = (E + 63) / 64;   // experts held per lane
  static_assert(E <= 128 && K <= 8, "");
  const __amdgpu_buffer_rsrc_t R = rsrc(p.rlog + (size_t)l * MAXB * E);
  float v[EPL];
#pragma unroll
  for (int k = 0; k < EPL; ++k) v[k] = (lane + 64 * k < E) ? ldc(R, 4u * (b * E + lane + 64 * k)) : -INFINITY;
  if (emit && p.rlog_out) {
#pragma unroll
    for (int k = 0; k < EPL; ++k)
      if (lane + 64 * k < E) p.rlog_out[((size_t)l * p.B + b) * E + lane + 64 * k] = v[k];
  }
  // radix select of the K-th largest order key T (a ballot per bit: no data leaves the lanes),
  // then every key above T and the lowest-indexed keys equal to T
  uint32_t key[EPL];
#pragma unroll
  for (int k = 0; k < EPL; ++k) {
    const uint32_t u = __float_as_uint(v[k] + 0.0f);          // -0 and +0 tie, as they compare
    key[k] = (lane + 64 * k < E) ? ((u & 0x80000000u) ? ~u : (u | 0x80000000u)) : 0u;
  }
  uint32_t T = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = T | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < EPL; ++k) cnt += __builtin_popcountll(__ballot(key[k] >= c));
    if (cnt >= K) T = c;
  }
  unsigned long long sel[2] = {0ull, 0ull};
  int need = K;
#pragma unroll
  for (int k = 0; k < EPL; ++k) {
    sel[k] = __ballot(key[k] > T);
    need -= __builtin_popcountll(sel[k]);
  }
#pragma unroll
  for (int k = 0; k < EPL; ++k) {
    unsigned long long eq = __ballot(key[k] == T);
    while (need > 0 && eq) { sel[k] |= eq & (~eq + 1); eq &= eq - 1; --need; }
  }
  m0 = sel[0];
  m1 = sel[1];
  // the selected experts in ascending index order (the MoE sum order) and their logits
  unsigned long long r0 = m0, r1 = m1;
#pragma unroll
  for (int i = 0; i < K; ++i) {
    const bool lo = r0 != 0;
    const unsigned long long r = lo ? r0 : r1;
    const int bitpos = __builtin_ctzll(r);
    if (lo) r0 &= r0 - 1; else r1 &= r1 - 1;
    widx[i] = bitpos + (lo ? 0 : 64);
    const float src = lo ? v[0] : v[EPL - 1];
    wval[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(src), bitpos));
  }
}

// Routing decision of layer l for the whole batch, computed by the last router tile (R7 of the
// oracle's readings): top-k of the raw logits with ties to the lower index, softmax over the k
// selected, the union of experts over the batch and each union slot's token list.
template <class S>
__device__ __forceinline__ void compute_route(CParams& p, int l) {
  constexpr int E = S::E, K = S::K;
  const int B = p.B;
  const int tx = tid(), lane = tx & 63, wave = __builtin_amdgcn_readfirstlane(tx >> 6);
  unsigned long long* mask = &ctl_s.mask[0][0];   // [MAXB][2] selected experts
  const __amdgpu_buffer_rsrc_t RT = rsrc(p.route + l);
  for (int b = wave; b < B; b += NWAVE) {
    int widx[K];
    float wval[K];
    unsigned long long m0, m1;
    topk_select<S>(p, l, b, lane, true, widx, wval, m0, m1);
    float top = wval[0];
#pragma unroll
    for (int i = 1; i < K; ++i) top = fmaxf(top, wval[i]);
    float ex[K];
#pragma unroll
    for (int i = 0; i < K; ++i) ex[i] = expf(wval[i] - top);
    float tot;
    if constexpr (K == 8) {
      tot = ((ex[0] + ex[1]) + (ex[2] + ex[3])) + ((ex[4] + ex[5]) + (ex[6] + ex[7]));
    } else {
      tot = 0.f;
#pragma unroll
      for (int i = 0; i < K; ++i) tot += ex[i];
    }
#pragma unroll
    for (int i = 0; i < K; ++i) {
      if (lane == i) {
        stci(RT, (uint32_t)offsetof(RouteTable, sel) + 4u * (b * 8 + i), widx[i]);
        stc(RT, (uint32_t)offsetof(RouteTable, w) + 4u * (b * 8 + i), ex[i] / tot);
        if (p.topk_out) p.topk_out[((size_t)l * B + b) * K + i] = widx[i];
      }
    }
    if (lane == 0) { mask[2 * b] = m0; mask[2 * b + 1] = m1; }
  }
  __syncthreads();
  // union over the batch (ascending expert ids) and each union slot's tokens (ascending b)
  if (tid() < E) {
    const int e = tid();
    unsigned long long u0 = 0, u1 = 0;
    for (int b = 0; b < B; ++b) { u0 |= mask[2 * b]; u1 |= mask[2 * b + 1]; }
    const bool used = e < 64 ? (u0 >> e) & 1 : (u1 >> (e - 64)) & 1;
    const int slot = e < 64 ? __builtin_popcountll(u0 & ((1ull << e) - 1))
                            : __builtin_popcountll(u0) + __builtin_popcountll(u1 & ((1ull << (e - 64)) - 1));
    if (e == E - 1) stci(RT, (uint32_t)offsetof(RouteTable, n_union), __builtin_popcountll(u0) + __builtin_popcountll(u1));
    if (used) {
      stci(RT, (uint32_t)offsetof(RouteTable, union_e) + 4u * slot, e);
      int nt = 0;
      for (int b = 0; b < B; ++b) {
        const unsigned long long b0 = mask[2 * b], b1 = mask[2 * b + 1];
        const bool has = e < 64 ? (b0 >> e) & 1 : (b1 >> (e - 64)) & 1;
        if (!has) continue;
        const int i = e < 64 ? __builtin_popcountll(b0 & ((1ull << e) - 1))
                             : __builtin_popcountll(b0) + __builtin_popcountll(b1 & ((1ull << (e - 64)) - 1));
        stci(RT, (uint32_t)offsetof(RouteTable, tok_bi) + 4u * (slot * MAXB + nt), (b << 8) | i);
        ++nt;
      }
      stci(RT, (uint32_t)offsetof(RouteTable, n_tok) + 4u * slot, nt);
    }
  }
}

template <class S, int TB>
__device__ __forceinline__ bool op_router(int task) {
  CParams& p = P();
  Ctl& ctl = ctl_s;
  float* sm = smem;
  const TaskHdr T = read_task(p, task);
  constexpr int H = S::H, E = S::E, KW = S::kw(H), NP = (Geo<KW>::CPL >= 4 || S::WF) ? 4 : 8;
  const auto& Lp = cst(p.layers)[T.layer];
  const int row0 = T.a0, nrows = T.a1;
  auto rowptr = [&](int r) { return Lp.w_router + (size_t)(row0 + r) * S::rw(H); };
  const bool pre = !(p.flags & 2);
  const __amdgpu_buffer_rsrc_t R = rsrc(p.rlog + (size_t)T.layer * MAXB * E);
  const float* bias = p.has_bias ? Lp.router_bias : nullptr;
  auto emit = [&](int r, int t, float v) {
    const int e = row0 + r;
    stc(R, 4u * (t * E + e), bias ? v + bias[e] : v);
  };
  if constexpr (TB > 1) {                        // several tokens: the matrix cores
    MRows<S> A;
    if (pre) mrows_load<S>(A, 0, nrows, rowptr);
    if (!wait_ge(p, ctl, T.w0, (uint32_t)T.t0, T.id)) return false;
    if (tid() < MAXB) ctl.toks[tid()] = tid();
    __syncthreads();
    stage_norm<S, MRows<S>::AS>(p, T.layer, ctl.toks, p.B, Lp.attn_norm, sm, T.id);
    MARK(0);
    mrows_stream<S>(A, pre, nrows, p.B, rowptr, sm, sm + MRows<S>::RED, emit);
  } else {
    WBuf<KW, NP, S::WF> A;
    if (pre) load_block<KW, NP, S::WF>(A, 0, nrows, rowptr);
    if (!wait_ge(p, ctl, T.w0, (uint32_t)T.t0, T.id)) return false;
    if (tid() < MAXB) ctl.toks[tid()] = tid();
    __syncthreads();
    stage_norm<S>(p, T.layer, ctl.toks, p.B, Lp.attn_norm, sm, T.id);
    MARK(0);
    gemv_stream<KW, NP, TB, (TB > 1 ? 2 : 1), S::WF>(A, pre, nrows, p.B, rowptr,
        [&](int r, int t) { return sm + (size_t)t * H; }, emit);
  }
  MARK(1);
  const uint32_t old = signal(p, ctl, T.sig, true);
  MARK(2);
  if (old + 1 == (uint32_t)T.a2) {      // last router tile of the layer: route the batch
    __syncthreads();
    compute_route<S>(p, T.layer);
    MARK(3);
    signal(p, ctl, T.sig2, false);
  }
  return true;
}

// Expert slice: rows f0..f0+nf of W_gate[e] and W_up[e] for the tokens routed to union slot u;
// h = SiLU(g) * u (P3 "Key Technologies and Architecture": fused SiLU-multiply). The normed input of
// every token is staged as soon as x_l is complete, before the routing decision is awaited, so
// that only the route table and the weights are on the path after the router.
template <class S, int TB>
__device__ __forceinline__ bool op_gateup(int task) {
  static_assert(TB * S::F <= TB * S::H, "down items stage h where the normed input lives");
  CParams& p = P();
  Ctl& ctl = ctl_s;
  float* sm = smem;
  const TaskHdr T = read_task(p, task);
  constexpr int H = S::H, F = S::F, K = S::K, KWH = S::kw(H), NP = (Geo<KWH>::CPL >= 4) ? 2 : 4;
  // bf16 rows of an item take the slot's tokens in pairs (each weight unpacked once per pair; the
  // same products in the same order). Measured on MI355X: batch 8 1179 -> 1195 tok/s, the ragged
  // Zipf-routed batch (hot experts with up to 8 tokens) 1353 -> 1442. FP8 and MXFP4 rows keep one
  // token at a time: pairs spill 74 and 346 registers in those instances.
  constexpr int TGE = (TB > 1 && S::WF == 0) ? 2 : 1;
  const int l = T.layer;
  const auto& Lp = cst(p.layers)[l];
  // Queue mode (a3 >= 0, P3 "Scheduling and Performance Benchmarks": dynamic work stealing): the
  // items (union slot u, FFN slice j) of the layer are drawn from counter a3, whose sub-counter q
  // hands out the items q, q + nq, q + 2 nq, ... (a0 = own sub-queue, a1 = nq, a2 = slices per
  // slot, a4 = rows per slice). The task draws from its own sub-queue until it is exhausted, then
  // steals from the next ones. The first draw is issued before the dependency waits.
  const bool dyn = T.a3 >= 0;
  const int nq = dyn ? T.a1 : 1;
  const int qd = dyn ? (T.a5 & 0xffff) : 0;   // down items per union slot (queue mode)
  const int n_oi = dyn ? (T.a5 >> 16) : 0;    // O-projection items after them (queue mode)
  const int tx = tid(), lane = tx & 63, wave = __builtin_amdgcn_readfirstlane(tx >> 6);
  int sq = dyn ? T.a0 : 0;
  // a draw: lane 0 of wave 0 takes the next item of sub-queue q; lanes < nq read every sub-queue's
  // head at the same time (a snapshot: heads only grow, so a sub-queue it shows exhausted stays so)
  uint32_t kreq = 0, head = 0xffffffffu;
  auto draw = [&](int q) {
    if (wave == 0) {
      if (lane == 0) kreq = ctr_add(ctr_at(p, T.a3, q), 1u);
      head = lane < nq ? ctr_load(ctr_at(p, T.a3, lane)) : 0xffffffffu;
    }
  };
  if (dyn) draw(sq);
  // the normed input of every token: staged once per worker and layer (consecutive expert tasks
  // of one layer on a worker reuse it), before the routing decision is awaited
  if (ctl.norm_l != l) {
    if (!wait_ge(p, ctl, T.w0, (uint32_t)T.t0, T.id)) return false;     // x_l complete
    if (tid() < MAXB) ctl.toks[tid()] = tid();
    __syncthreads();
    stage_norm<S>(p, l, ctl.toks, p.B, Lp.attn_norm, sm, T.id);       // act[b] for every batch row
    if (tid() == 0) ctl.norm_l = l;
  }
  MARK(0);
  if (!wait_ge(p, ctl, T.w1, (uint32_t)T.t1, T.id)) return false;     // every router tile done
  // the routing decision, taken here from the logits with the same selection as the route table
  // (no further hop through the router's last tile): each wave selects for its tokens
  for (int b = wave; b < p.B; b += NWAVE) {
    int widx[K];
    float wval[K];
    unsigned long long m0, m1;
    topk_select<S>(p, l, b, lane, false, widx, wval, m0, m1);
    if (lane == 0) { ctl.mask[b][0] = m0; ctl.mask[b][1] = m1; }
  }
  __syncthreads();
  unsigned long long u0 = 0, u1 = 0;
  for (int b = 0; b < p.B; ++b) { u0 |= ctl.mask[b][0]; u1 |= ctl.mask[b][1]; }
  const int n0 = __builtin_popcountll(u0), nu = n0 + __builtin_popcountll(u1);
  // expert of union slot u (the u-th selected expert in ascending order); thread 0 lists its tokens
  // (batch row, rank of the expert in that token's selection) in ctl.toks / ctl.trank, ctl.flag
  auto expert_of = [&](int u) {
    unsigned long long m = u < n0 ? u0 : u1;
    for (int j = u < n0 ? u : u - n0; j > 0; --j) m &= m - 1;
    return (u < n0 ? 0 : 64) + __builtin_ctzll(m);
  };
  auto slot_expert = [&](int u) {
    const int e = expert_of(u);
    if (tx == 0) {
      int nt = 0;
      for (int b = 0; b < p.B; ++b) {
        const unsigned long long b0 = ctl.mask[b][0], b1 = ctl.mask[b][1];
        const bool has = e < 64 ? (b0 >> e) & 1 : (b1 >> (e - 64)) & 1;
        if (!has) continue;
        ctl.toks[nt] = b;
        ctl.trank[nt] = e < 64 ? __builtin_popcountll(b0 & ((1ull << e) - 1))
                               : __builtin_popcountll(b0) + __builtin_popcountll(b1 & ((1ull << (e - 64)) - 1));
        ++nt;
      }
      ctl.flag = nt;
    }
    return e;
  };
  // the 2 nf rows of an item: W_gate[e] rows f0.., then W_up[e] rows f0..
  auto gu_rows = [&](int e, int f0, int nf) {
    const uint16_t* wg = Lp.w_gate + (size_t)e * F * S::rw(H);
    const uint16_t* wu = Lp.w_up + (size_t)e * F * S::rw(H);
    return [=](int r) { return r < nf ? wg + (size_t)(f0 + r) * S::rw(H) : wu + (size_t)(f0 + r - nf) * S::rw(H); };
  };
  int slices_c = 1, rows = 1, n_gu = 0, n_items = 0;   // the queue's item geometry (queue mode)
  // hand the draw to the workgroup, with the sub-queue that had the most items left in the
  // snapshot (-1: none had any)
  auto publish = [&]() {
    if (wave == 0) {
      const int64_t first = (int64_t)head * nq + lane;
      const int rem = lane < nq && first < n_items ? (int)((n_items - first + nq - 1) / nq) : 0;
      const int best = (int)wmax<64>((float)rem);
      const unsigned long long who = __ballot(rem == best && rem > 0);
      if (lane == 0) {
        ctl.item = (int)kreq;
        ctl.steal = who ? __builtin_ctzll(who) : -1;
      }
    }
    __syncthreads();
  };
  // rows f0..f0+nf of union slot u for its tokens. A holds the item's first weight block when
  // `loaded` (requested by the previous item). With `chain` (queue mode), once the item's weights
  // are consumed the next draw is published and, when it is a gate/up item, its first weight block
  // is requested before this item's stores and drain, so that the worker never waits a whole memory
  // round trip between two items. Returns whether it did.
  auto run_item = [&](int u, int f0, int nf, WBuf<KWH, NP, S::WF>& A, bool loaded, bool chain) -> bool {
    if (ctl.norm_l != l) {       // a down item used the staging area since: stage the normed input again
      __syncthreads();
      if (tid() < MAXB) ctl.toks[tid()] = tid();
      __syncthreads();
      stage_norm<S>(p, l, ctl.toks, p.B, Lp.attn_norm, sm, T.id);
      if (tid() == 0) ctl.norm_l = l;
      __syncthreads();
    }
    const int e = slot_expert(u);
    const auto rowptr = gu_rows(e, f0, nf);
    if (!loaded) load_block<KWH, NP, S::WF>(A, 0, 2 * nf, rowptr);
    __syncthreads();
    const int ntok = ctl.flag;
    MARK(1);
    int brow[TB];       // act row (batch row) of the slot's t-th token
#pragma unroll
    for (int t = 0; t < TB; ++t) brow[t] = t < ntok ? ctl.toks[t] : 0;
    float* gu = sm + (size_t)TB * H;                 // [TB][2 nf]
    gemv_stream<KWH, NP, TB, TGE, S::WF>(A, true, 2 * nf, ntok, rowptr,
        [&](int r, int t) { return sm + (size_t)brow[t] * H; },
        [&](int r, int t, float v) { gu[t * 2 * nf + r] = v; });
    bool next = false;
    if (chain) {
      publish();                           // (a barrier: gu is complete too)
      const int in = sq + nq * ctl.item;
      if (in < n_gu) {
        const int un = in / slices_c, fn = (in - un * slices_c) * rows, nfn = F - fn < rows ? F - fn : rows;
        load_block<KWH, NP, S::WF>(A, 0, 2 * nfn, gu_rows(expert_of(un), fn, nfn));
        next = true;
      }
    } else {
      __syncthreads();
    }
    MARK(2);
    const __amdgpu_buffer_rsrc_t Hb = rsrc(p.h + (size_t)l * MAXB * K * F);
    for (int i = tid(); i < ntok * nf; i += NT) {
      const int t = i / nf, f = i % nf;
      const float g = gu[t * 2 * nf + f], up = gu[t * 2 * nf + nf + f];
      const float hv = (g / (1.f + expf(-g))) * up;
      stc(Hb, 4u * ((ctl.toks[t] * K + ctl.trank[t]) * F + f0 + f), hv);
    }
    if (qd > 0) {
      // one more finished gate/up item of slot u: its h rows are visible before the count moves
      drain();
      __syncthreads();
      if (tx == 0) ctr_add(p.slot_ctr + ((size_t)l * MAX_SLOTS + u) * CTR_STRIDE, 1u);
    }
    __syncthreads();      // toks / trank / gu are rewritten by the next item
    return next;
  };
  // down item q of union slot u: rows q*DOWN_ROWS.. of W_down[e] for every token of the slot, once
  // every gate/up item of the slot is done: y[b][rank][row] = W_down[e][row] . h[b][rank]. Its weight
  // rows are requested before the slot's count is awaited. The staged h overwrites the normed input.
  auto run_down = [&](int u, int q) -> bool {
    // (MXFP4: two passes of 8 rows per wave - a block of the same 64 rows' bytes, half the registers)
    constexpr int NPD = S::WF == 2 ? 2 : 4;
    const int e = slot_expert(u);
    const int row0 = q * DOWN_ROWS, nr = H - row0 < DOWN_ROWS ? H - row0 : DOWN_ROWS;
    const uint16_t* wd = Lp.w_down + ((size_t)e * H + row0) * S::rw(F);
    auto rowptr = [&](int r) { return wd + (size_t)r * S::rw(F); };
    WBuf<S::kw(F), NPD, S::WF> A;
    load_block<S::kw(F), NPD, S::WF>(A, 0, nr, rowptr);
    if (tid() == 0) ctl.norm_l = -1;
    __syncthreads();
    const int ntok = ctl.flag;
    int yoff[TB], hoff[TB];
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      const int bt = t < ntok ? ctl.toks[t] : 0, rk = t < ntok ? ctl.trank[t] : 0;
      yoff[t] = (bt * K + rk) * H + row0;
      hoff[t] = (bt * K + rk) * F;
    }
    if (!wait_word(p, ctl, p.slot_ctr + ((size_t)l * MAX_SLOTS + u) * CTR_STRIDE, (uint32_t)slices_c, T.id, (uint32_t)u))
      return false;
    // h of every token of the slot into LDS: all loads first, then the writes
    const __amdgpu_buffer_rsrc_t Hr = rsrc(p.h + (size_t)l * MAXB * K * F);
    constexpr int NI = (TB * F + 4 * NT - 1) / (4 * NT);
    f4 hv[NI];
#pragma unroll
    for (int v = 0; v < NI; ++v) {
      const int idx = (v * NT + tx) * 4, t = idx / F, f = idx - t * F;
      int ho = 0;
#pragma unroll
      for (int tt = 0; tt < TB; ++tt) if (tt == t) ho = hoff[tt];
      hv[v] = t < ntok ? ldc4(Hr, 4u * (ho + f)) : f4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int v = 0; v < NI; ++v) {
      const int idx = (v * NT + tx) * 4, t = idx / F;
      if (t < ntok) *reinterpret_cast<f4*>(sm + idx) = hv[v];
    }
    __syncthreads();
    MARK(5);
    const __amdgpu_buffer_rsrc_t Y = rsrc(p.y + (size_t)l * MAXB * K * H);
    gemv_stream<S::kw(F), NPD, TB, TGE, S::WF>(A, true, nr, ntok, rowptr,
        [&](int r, int t) { return sm + (size_t)t * F; },
        [&](int r, int t, float v) {
          int yo = 0;
#pragma unroll
          for (int tt = 0; tt < TB; ++tt) if (tt == t) yo = yoff[tt];
          stc(Y, 4u * (yo + r), v);
        });
    MARK(6);
    __syncthreads();      // toks / trank / the staged h are rewritten by the next item
    return true;
  };
  // O-projection item j (between the gate/up and the down items): rows of W_o for a group of OQT
  // tokens, o[l][b][row] = W_o[row] . attn[b], once every attention merge of the layer is in (the
  // attention counter is the one allocated right before the queue's); the output rows add it
  // afterwards. Item j is row block j / ntg for token group j % ntg (ntg groups of OQT tokens), so an
  // item stages its tokens' attention once. One row pass per block (the register budget of this op);
  // bf16 rows take the group's tokens in pairs (batch 8 1190 -> 1195, ragged 1433 -> 1446 tok/s).
  constexpr int OQT = 4;
  auto run_oproj = [&](int j, int orows, int ntg) -> bool {
    constexpr int AD = S::AD;
    constexpr int NSL = S::HPG * S::D / 256 > 1 ? S::HPG * S::D / 256 : 1;   // merges per (token, group)
    const int rb = j / ntg, b0 = (j - rb * ntg) * OQT;
    const int r0 = rb * orows, nr = H - r0 < orows ? H - r0 : orows;
    const int nt = p.B - b0 < OQT ? p.B - b0 : OQT;
    if (nr <= 0 || nt <= 0) return true;     // (no rows or tokens left for this item)
    auto orow = [&](int r) { return Lp.w_o + (size_t)(r0 + r) * S::rw(AD); };
    WBuf<S::kw(AD), 1, S::WF> A;
    load_block<S::kw(AD), 1, S::WF>(A, 0, nr, orow);
    if (tid() == 0) ctl.norm_l = -1;     // the staged normed input is overwritten below
    if (!wait_ge(p, ctl, T.a3 - 1, (uint32_t)(p.B * S::HKV * NSL), T.id)) return false;
    const __amdgpu_buffer_rsrc_t At = rsrc(p.attn + (size_t)l * MAXB * AD);
    const __amdgpu_buffer_rsrc_t Ob = rsrc(p.o + (size_t)l * MAXB * H);
    __syncthreads();                     // every wave is done with the previous item's LDS
    stage_f4<OQT * AD>(sm, At, 4u * (b0 * AD), nt * AD);
    __syncthreads();
    gemv_stream<S::kw(AD), 1, OQT, (S::WF == 0 ? 2 : TG_ROWS<S>), S::WF>(A, true, nr, nt, orow,
        [&](int r, int t) { return sm + (size_t)t * AD; },
        [&](int r, int t, float v) { stc(Ob, 4u * ((b0 + t) * H + r0 + r), v); });
    __syncthreads();                     // the staging area is free for the next item
    return true;
  };
  if (TB == 1 || !dyn) {           // one token: static slices only (the queue is never scheduled)
    if (T.a0 < nu) {
      WBuf<KWH, NP, S::WF> A;
      run_item(T.a0, T.a1, T.a2, A, false, false);
    }
  } else if constexpr (TB > 1) {
    // item size from the step's union: with at least four slices per worker, a draw takes three
    // adjacent slices (two for MXFP4 rows, whose decode makes an item's bytes slower to consume) -
    // fewer draws and longer streams; a small union (skewed routing) keeps single slices so that the
    // work spreads over more workers. Every task derives the same grain. Measured on MI355X (batch 8,
    // 8K context, tok/s): bf16 1165 / 1183 / 1157 and FP8 1274 / 1288 / 1231 with two / three /
    // four slices, MXFP4 1201 / 1188 with two / three; grain 2 under skewed routing: 1278 vs 1361.
    constexpr int GMAX = S::WF == 2 ? 2 : 3;
    const int slices = T.a2, nfs = T.a4;
    const int grain = (nu * slices >= 4 * p.n_workers && GMAX * nfs <= 48) ? GMAX : 1;
    slices_c = (slices + grain - 1) / grain;
    rows = grain * nfs;
    n_gu = nu * slices_c;                           // gate/up items first, then the down items,
    const int n_dn = n_gu + nu * qd;                // then the O-projection items
    n_items = n_dn + n_oi;
    const int ntg = (p.B + OQT - 1) / OQT;          // token groups of the O-projection items
    const int orows = n_oi > 0 ? (H + n_oi / ntg - 1) / (n_oi / ntg) : 0;
    publish();
    int probes = 1;
    bool more = true;
    {
      // the gate/up items, which head every sub-queue: each one requests the next one's first
      // weight block (A stays in registers from one item to the next)
      WBuf<KWH, NP, S::WF> A;
      bool pre = false;
      for (;;) {
        const int k = ctl.item, steal_q = ctl.steal;
        __syncthreads();    // every thread has read the draw
        const int i = sq + nq * k;
        if (i >= n_items) {               // this sub-queue is exhausted: steal from another one
          if (steal_q < 0 || probes >= STEAL_PROBES) { more = false; break; }
          ++probes;
          sq = steal_q;
          draw(sq);
          publish();
          continue;
        }
        if (i >= n_gu) break;             // (the draw stays published for the loop below)
        draw(sq);                         // the next draw, in flight during the item
        const int u = i / slices_c, f0 = (i - u * slices_c) * rows;
        pre = run_item(u, f0, F - f0 < rows ? F - f0 : rows, A, pre, true);
      }
    }
    while (more) {
      const int k = ctl.item, steal_q = ctl.steal;
      __syncthreads();    // every thread has read the draw
      const int i = sq + nq * k;
      if (i >= n_items) {               // this sub-queue is exhausted: steal from another one
        if (steal_q < 0 || probes >= STEAL_PROBES) break;
        ++probes;
        sq = steal_q;
        draw(sq);
        publish();
        continue;
      }
      draw(sq);                         // the next draw, in flight during the item
      if (i < n_gu) {                   // (a stolen gate/up item after the sub-queue's others)
        const int u = i / slices_c, f0 = (i - u * slices_c) * rows;
        WBuf<KWH, NP, S::WF> A;
        run_item(u, f0, F - f0 < rows ? F - f0 : rows, A, false, false);
      } else if (i >= n_gu + n_oi) {
        const int i2 = i - n_gu - n_oi, u = i2 / qd;
        if (!run_down(u, i2 - u * qd)) return false;
      } else {
        // (compiled for bf16 and MXFP4 matrices: in the FP8 instances the extra GEMV path costs 15
        // more spilled registers, and the schedule gives them no such items)
        if constexpr (S::WF != 1) {
          if (!run_oproj(i - n_gu, orows, ntg)) return false;
        } else {
          return false;                  // (the host's validator refuses such a schedule)
        }
      }
      publish();
    }
  }
  MARK(4);
  drain_t(p);
  MARK(3);
  signal(p, ctl, T.sig, false);
  return true;
}

// Split-KV paged GQA decode attention for one (sequence b, KV group g, key range) with fused RoPE
// (P3 "Key Technologies and Architecture": restructured paged attention, fused RoPE; P1 "From
// demo to a full serving system": paged KV, ragged lengths). The split holding the new position
// writes the new K/V into the cache and scores it in fp32 against the rounded key. Each split
// publishes an unnormalised partial (m, l, o) and bumps its group's arrival counter; merge tasks
// combine the partials.
//
// Both contractions run on the matrix cores (16x16x32 bf16 MFMA). Scores S = Q K^T per block of
// 16 keys (one KV page, 4 KB contiguous), the A rows being the group's HPG query heads split into
// bf16 high and low parts (q = hi + lo to 2^-16), so fp32 accuracy is kept. P V per 32-key block,
// with P split the same way and V transposed through a per-wave LDS tile. The first 256-key chunk
// of K and V is requested before the dependency wait.

// LDS layout of an attention task, in floats (every region 16-byte aligned)
template <class S>
struct AttnLds {
  static constexpr int al(int x) { return (x + 3) & ~3; }
  static constexpr int D = S::D, HPG = S::HPG;
  static constexpr int PS = SPLIT_MAX + 32;        // P row stride (keys, zero tail for the last block)
  static constexpr int VRS = D / 2 + 4;            // V tile row stride in floats (bf16 pairs + pad)
  static constexpr int SB = 0;                     // [HPG][PS] scores -> probabilities
  static constexpr int VT = al(SB + HPG * PS);     // [NWAVE][32][VRS] V tiles (one per wave)
  static constexpr int OB = VT;                    // [NWAVE][HPG][D] per-wave P V, after the tiles
  static constexpr int VN = al(VT + (NWAVE * 32 * VRS > NWAVE * HPG * D ? NWAVE * 32 * VRS : NWAVE * HPG * D));
  static constexpr int ML = al(VN + D);
  static constexpr int PG = al(ML + 2 * HPG);
  static constexpr int KN = al(PG + SPLIT_MAX / PAGE + 1);
  static constexpr int QF = al(KN + D / 2);
  static constexpr int END = al(QF + HPG * D);
};


template <class S>
struct OutLds {   // LDS layout of a batched output task, in floats
  static constexpr int KF = S::K * S::F;
  static constexpr int A = 0;                           // [OUT_OT][AD] attention (O-projection phase)
  static constexpr int HA = 0, HB = KF;                 // [K][F] h of two tokens (MoE phase)
  static constexpr int Y = (OUT_OT * S::AD > 2 * KF ? OUT_OT * S::AD : 2 * KF);   // [K][OUT_MAXR]
  static constexpr int MO = Y + S::K * OUT_MAXR;        // [MAXB][OUT_MAXR] MoE term
  static constexpr int XV = MO + MAXB * OUT_MAXR;       // [MAXB][OUT_MAXR] x_l rows
  static constexpr int O = XV + MAXB * OUT_MAXR;        // [OUT_OT][OUT_MAXR] O-projection rows
  static constexpr int END = O + OUT_OT * OUT_MAXR;
};

// Dynamic LDS: the ops' working area (the largest of: norm-staged activations + GEMV scratch,
// attention buffers, OUT staging, routing scratch), then the step's RoPE table.
template <class S>
__host__ __device__ constexpr int rope_off(int tb) {
  int act = tb * S::H + tb * 2 * 64 + 1024;
  if (tb > 1 && MRows<S>::END + 256 > act) act = MRows<S>::END + 256;   // matrix-core staging + argmax
  const int att = AttnLds<S>::END;
  const int out1 = S::AD + S::K * S::F + OUT_MAXR + S::K * OUT_MAXR + 2 * MAXB * OUT_MAXR;
  const int out = tb > 1 && OutLds<S>::END > out1 ? OutLds<S>::END : out1;
  const int rte = MAXB * S::E * 3 + S::E + 64;
  const int mrg = MERGE_MAX * 2 * 2 * NWAVE + 2 * NWAVE;
  int m = act;
  if (att > m) m = att;
  if (out > m) m = out;
  if (rte > m) m = rte;
  if (mrg > m) m = mrg;
  return (m + 63) & ~63;
}

// cos and sin of pos_b * inv_freq[i] for every sequence b of the step: [b][0..D/2) cos, [D/2..D) sin
template <class S, int TB>
__device__ __forceinline__ float* rope_tab() { return smem + rope_off<S>(TB); }

template <class S, int TB, int VAR>
__device__ __forceinline__ bool op_attn(int task) {
  CParams& p = P();
  Ctl& ctl = ctl_s;
  float* sm = smem;
  const TaskHdr T = read_task(p, task);
  typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
  constexpr int D = S::D, HPG = S::HPG, LPK = D / 8, KPW = 64 / LPK, KPI = NWAVE * KPW;
  constexpr int KB = D / 32;             // MFMA k-blocks per head vector
  constexpr int KC = 256;                // keys per chunk
  constexpr int GPW = KC / 16 / NWAVE;   // 16-key column blocks per wave per chunk
  constexpr int VPL = KC / KPI;          // V loads per lane per chunk (P V layout)
  static_assert(2 * HPG <= 16 && HPG % 2 == 0 && D % 32 == 0 && KC % KPI == 0, "");
  static_assert(KC / NWAVE == 64 && KPW * VPL == 64 && HPG <= 2 * NWAVE, "P V: one 64-key quarter per wave");
  const int l = T.layer, b = T.a0, g = T.a1, k0 = T.a2, k1 = T.a3;
  const int pbase = T.a4, s_idx = T.a5 & 0xffff, nsplit = T.a5 >> 16;
  const auto& Lp = cst(p.layers)[l];
  const int tx = tid(), lane = tx & 63, wave = __builtin_amdgcn_readfirstlane(tx >> 6);
  const int li = lane % LPK;                                    // 8-dim chunk of a V row
  const int col = lane & 15, grp = lane >> 4;                   // MFMA layout
  const int n_ctx = cst(p.seq_lens)[b], pos = cst(p.positions)[b];
  const bool last = k1 < 0;
  if (pos != n_ctx - 1 || pos < 0 || n_ctx > p.max_pages * PAGE) {
    if (tx == 0) raise_error(p, DEV_BAD_POS, T.id, -1, (uint32_t)n_ctx, (uint32_t)pos, (uint32_t)b);
    return false;
  }
  int kend = last ? pos : (k1 < pos ? k1 : pos);
  if (kend < k0) kend = k0;
  const int nk = kend - k0;                       // cached keys scored by this task
  const int ntot = nk + (last ? 1 : 0);
  if ((last && pos < k0) || ntot > SPLIT_MAX) {
    if (tx == 0) raise_error(p, DEV_STALE, T.id, -1, (uint32_t)k0, (uint32_t)pos, (uint32_t)b);
    return false;
  }
  // LDS layout (float offsets in AttnLds<S>)
  using L = AttnLds<S>;
  const float* cs = rope_tab<S, TB>() + b * D;     // [D/2] cos, [D/2] sin at pos
  constexpr int PS = L::PS, VRS = L::VRS;
  float* sbuf = sm + L::SB;                        // [HPG][PS] scores -> probabilities
  uint32_t* vt = reinterpret_cast<uint32_t*>(sm + L::VT) + wave * 32 * VRS;   // this wave's V tile
  float* vnew = sm + L::VN;                        // [D]
  float* ml = sm + L::ML;                          // [2][HPG]
  float* obuf = sm + L::OB;                        // [NWAVE][HPG][D]
  int* pg = reinterpret_cast<int*>(sm + L::PG);    // [SPLIT_MAX / PAGE + 1] page ids
  uint32_t* knew = reinterpret_cast<uint32_t*>(sm + L::KN);   // [D / 2] new key, bf16 pairs
  float* qf = sm + L::QF;                          // [HPG][D] RoPE'd queries
  {
    const __attribute__((address_space(4))) int32_t* bt = cst(p.block_tables) + (size_t)b * p.max_pages + k0 / PAGE;
    const int npg = (ntot + PAGE - 1) / PAGE;
    for (int i = tx; i < npg; i += NT) {
      int page = bt[i];
      if (page < 0 || page >= p.num_pages) {
        raise_error(p, DEV_BAD_PAGE, T.id, -1, (uint32_t)p.num_pages, (uint32_t)page, (uint32_t)(k0 / PAGE + i));
        page = 0;
      }
      pg[i] = page;
    }
  }
  __syncthreads();
  // key j, dims d0..d0+7 -> element offset in the K (or V) cache
  auto kaddr = [&](int j, int d0) -> size_t {
    return (((size_t)pg[(j - k0) / PAGE] * S::HKV + g) * PAGE + (j % PAGE)) * D + d0;
  };
  const int nchunk = (nk + KC - 1) / KC;           // chunks of cached keys (the new key is apart)
  u4 kr[GPW][KB];       // MFMA B operands: key k0 + c*KC + (wave + NWAVE*i)*16 + col, dims 32kb + 8grp
  auto load_k = [&](int c) {
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
      const int j = k0 + c * KC + (wave + NWAVE * i) * 16 + col;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        kr[i][kb] = (j < kend) ? ldw(Lp.k_cache + kaddr(j, 32 * kb + 8 * grp)) : u4{0u, 0u, 0u, 0u};
    }
  };
  u4 vr[VPL];           // key k0 + c*KC + 64*wave + KPW*q + lane/LPK (the wave's quarter), dims 8li
  auto load_v = [&](int c) {
#pragma unroll
    for (int q = 0; q < VPL; ++q) {
      const int j = k0 + c * KC + (KC / NWAVE) * wave + KPW * q + lane / LPK;
      vr[q] = (j < kend) ? ldw(Lp.v_cache + kaddr(j, 8 * li)) : u4{0u, 0u, 0u, 0u};
    }
  };
  // the cached keys and values do not depend on this step's activations: the first chunk of both
  // is in flight while the task waits for the QKV rows. When a second chunk holds at most one page
  // (splits a little longer than a chunk), that page's values are requested with the first chunk:
  // they fall in wave 0's first rows, which take them in a few more registers instead of paying a
  // dependent round trip in the P V pass. (Its keys go to wave 0's first key registers once that
  // block's first-chunk products are done: holding them from the start as well would exceed the
  // register budget.)
  // (When the QKV tasks publish the step's keys - rows of one sequence in one step - keys of this
  // step's other rows may lie in the range, so nothing is read before the wait.)
  if constexpr (VAR == 2)
    if (!wait_ge(p, ctl, T.w0, (uint32_t)T.t0, T.id)) return false;
  load_k(0);
  load_v(0);
  const bool tail = nchunk == 2 && nk - KC <= PAGE;    // uniform in the workgroup
  constexpr int VT_Q = PAGE / KPW;                     // V loads of wave 0 that hold the tail page
  u4 vtl[VT_Q];
  if (tail && wave == 0) {
#pragma unroll
    for (int q = 0; q < VT_Q; ++q) {
      const int jv = k0 + KC + KPW * q + lane / LPK;
      vtl[q] = jv < kend ? ldw(Lp.v_cache + kaddr(jv, 8 * li)) : u4{0u, 0u, 0u, 0u};
    }
  }
  if constexpr (VAR != 2)
    if (!wait_ge(p, ctl, T.w0, (uint32_t)T.t0, T.id)) return false;
  const __amdgpu_buffer_rsrc_t Q = rsrc(p.qkv + ((size_t)l * MAXB + b) * S::QKVR);
  const float rsd = 1.0f / sqrtf((float)D);
  // rotate-half RoPE of 4 dims d0..d0+3 (all on one side of D/2) given x and its partner dims y
  auto rope4 = [&](f4 x, f4 y, int d0) -> f4 {
    f4 r;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int i = (d0 + m) % (D / 2);
      const float c = cs[i], s = cs[D / 2 + i];
      r[m] = d0 < D / 2 ? x[m] * c - y[m] * s : x[m] * c + y[m] * s;
    }
    return r;
  };
  // the group's query rows, RoPE'd, into LDS (one round trip); the last split also forms the new
  // key and value: RoPE(k) and v rounded to bf16 (the cache format), written at slot pos and kept in
  // LDS for scoring and for P V
  for (int i4 = 4 * tx; i4 < HPG * D; i4 += 4 * NT) {
    const int hh = i4 / D, d0 = i4 % D, pd0 = d0 < D / 2 ? d0 + D / 2 : d0 - D / 2;
    const uint32_t base = (uint32_t)((g * HPG + hh) * D);
    const f4 x = ldc4(Q, 4u * (base + d0)), y = ldc4(Q, 4u * (base + pd0));
    *reinterpret_cast<f4*>(qf + i4) = rope4(x, y, d0);
  }
  if (last && wave == 0 && lane < LPK) {
    const int d0 = 8 * li, pd0 = d0 < D / 2 ? d0 + D / 2 : d0 - D / 2;
    const uint32_t kbase = (uint32_t)(S::HQ * D + g * D), vbase = (uint32_t)((S::HQ + S::HKV) * D + g * D);
    const f4 x0 = ldc4(Q, 4u * (kbase + d0)), x1 = ldc4(Q, 4u * (kbase + d0 + 4));
    const f4 y0 = ldc4(Q, 4u * (kbase + pd0)), y1 = ldc4(Q, 4u * (kbase + pd0 + 4));
    const f4 v0 = ldc4(Q, 4u * (vbase + d0)), v1 = ldc4(Q, 4u * (vbase + d0 + 4));
    const f4 k0r = rope4(x0, y0, d0), k1r = rope4(x1, y1, d0 + 4);
    const float kk[8] = {k0r.x, k0r.y, k0r.z, k0r.w, k1r.x, k1r.y, k1r.z, k1r.w};
    const float vv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    uint32_t kw[4], vw[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t ka = f2bf(kk[2 * m]), kb2 = f2bf(kk[2 * m + 1]);
      const uint32_t va = f2bf(vv[2 * m]), vb2 = f2bf(vv[2 * m + 1]);
      kw[m] = ka | (kb2 << 16);
      vw[m] = va | (vb2 << 16);
      knew[4 * li + m] = kw[m];
      vnew[8 * li + 2 * m] = bf1((uint16_t)va); vnew[8 * li + 2 * m + 1] = bf1((uint16_t)vb2);
    }
    if constexpr (VAR != 2) {            // (else the QKV tasks have written them)
      const size_t off = kaddr(pos, 8 * li);
      *reinterpret_cast<u4*>(Lp.k_cache + off) = u4{kw[0], kw[1], kw[2], kw[3]};
      *reinterpret_cast<u4*>(Lp.v_cache + off) = u4{vw[0], vw[1], vw[2], vw[3]};
    }
  }
  __syncthreads();
  // MFMA A operand, row r = col: with a = r / 4, rows 4a, 4a+1 hold the bf16 high parts of heads
  // 2a, 2a+1 and rows 4a+2, 4a+3 their low parts (q - bf16(q)), so that the output rows a lane holds
  // (4 grp .. 4 grp + 3) are the two parts of heads 2 grp and 2 grp + 1
  bf8 qa[KB];
  {
    const int h = 2 * (col >> 2) + (col & 1);
    const bool valid = h < HPG, lo = (col & 2) != 0;
    const float* qrow = qf + (valid ? h : 0) * D + 8 * grp;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const f4 x0 = *reinterpret_cast<const f4*>(qrow + 32 * kb), x1 = *reinterpret_cast<const f4*>(qrow + 32 * kb + 4);
      const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      uint32_t w[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        uint32_t a = f2bf(x[2 * m]), c = f2bf(x[2 * m + 1]);
        if (lo) { a = f2bf(x[2 * m] - bf1((uint16_t)a)); c = f2bf(x[2 * m + 1] - bf1((uint16_t)c)); }
        w[m] = valid ? (a | (c << 16)) : 0u;
      }
      qa[kb] = __builtin_bit_cast(bf8, u4{w[0], w[1], w[2], w[3]});
    }
  }
  MARK(0);
  // ---- pass A: s[j][hh] = (k_j . q_hh) / sqrt(D) on the matrix cores, cached keys j < nk
  for (int c = 0; c < nchunk; ++c) {
    // a one-page second chunk is wave 0's first block only: its keys were requested into kr[0]
    // right after that block's first-chunk products (below)
    if (c > 0 && !tail) load_k(c);
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
      const int jb = c * KC + (wave + NWAVE * i) * 16;   // first key of the block, relative to k0
      if (jb >= nk) continue;                             // uniform in the wave
      f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kb], __builtin_bit_cast(bf8, kr[i][kb]), acc, 0, 0, 0);
      if (i == 0 && c == 0 && tail && wave == 0) {
        const int jk = k0 + KC + col;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          kr[0][kb] = jk < kend ? ldw(Lp.k_cache + kaddr(jk, 32 * kb + 8 * grp)) : u4{0u, 0u, 0u, 0u};
      }
      if (2 * grp < HPG && jb + col < nk) {
        sbuf[(2 * grp) * PS + jb + col] = (acc[0] + acc[2]) * rsd;
        sbuf[(2 * grp + 1) * PS + jb + col] = (acc[1] + acc[3]) * rsd;
      }
    }
  }
  __syncthreads();
  MARK(1);
  // ---- softmax statistics per head (half a wave per head, lanes over keys); the new key's score
  // is a plain fp32 dot product of the RoPE'd query with the bf16 key
  {
    const int hh = 2 * wave + (lane >> 5), sl = lane & 31;
    const bool hv = hh < HPG;
    float* prow = sbuf + (hv ? hh : 0) * PS;
    float snew = -INFINITY;
    if (last) {
      float t = 0.f;
      if (hv)
        for (int d2 = sl; d2 < D / 2; d2 += 32) {
          const uint32_t kw = knew[d2];
          t += qf[hh * D + 2 * d2] * bf_lo(kw) + qf[hh * D + 2 * d2 + 1] * bf_hi(kw);
        }
      snew = wsum<32>(t) * rsd;
    }
    // 256 keys per pass: each lane reads 8 consecutive keys as two 16-byte LDS reads (entries
    // past nk are masked; the buffer has room for them)
    float m = snew;
    if (hv)
      for (int j0 = 0; j0 < nk; j0 += 256) {
        const int jl = j0 + 8 * sl;
        const f4 va = *reinterpret_cast<const f4*>(prow + jl), vb = *reinterpret_cast<const f4*>(prow + jl + 4);
        const float v[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
#pragma unroll
        for (int u = 0; u < 8; ++u) m = jl + u < nk ? fmaxf(m, v[u]) : m;
      }
    m = wmax<32>(m);
    float lsum = 0.f;
    if (hv)
      for (int j0 = 0; j0 < nk; j0 += 256) {
        const int jl = j0 + 8 * sl;
        const f4 va = *reinterpret_cast<const f4*>(prow + jl), vb = *reinterpret_cast<const f4*>(prow + jl + 4);
        const float v[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
        float e[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          e[u] = jl + u < nk ? expf(v[u] - m) : 0.f;
          lsum += e[u];
        }
        if (jl < nk) {     // entries past nk are rewritten below (zeros and the new key)
          *reinterpret_cast<f4*>(prow + jl) = f4{e[0], e[1], e[2], e[3]};
          *reinterpret_cast<f4*>(prow + jl + 4) = f4{e[4], e[5], e[6], e[7]};
        }
      }
    lsum = wsum<32>(lsum);
    if (hv) {
      // the new key's probability, then zeros up to the end of the last 32-key block (P V reads it)
      const int zend = ((nk + 31) & ~31) + 32;
      for (int j = nk + sl; j < zend; j += 32) prow[j] = (last && j == nk) ? expf(snew - m) : 0.f;
      if (sl == 0) {
        ml[hh] = m;
        ml[HPG + hh] = last ? lsum + expf(snew - m) : lsum;
      }
    }
  }
  __syncthreads();
  MARK(2);
  // ---- pass B: o[hh][d] = sum_j p[hh][j] v_j[d] on the matrix cores. Each wave owns a 64-key
  // quarter of every chunk: its V rows go through a private LDS tile so that the B operand (8
  // consecutive keys of one dimension) is read column-wise; the A operand is P in bf16 high and low
  // parts, rows arranged as for the scores (heads 2a, 2a+1 high in rows 4a, 4a+1, low in 4a+2, 4a+3).
  constexpr int NCB = D / 16;            // 16-dim column blocks
  f4 oacc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) oacc[cb] = f4{0.f, 0.f, 0.f, 0.f};
  {
    const int ph = 2 * (col >> 2) + (col & 1);
    const bool pvalid = ph < HPG, plo = (col & 2) != 0;
    const float* prow = sbuf + (pvalid ? ph : 0) * PS;
    for (int c = 0; c < nchunk; ++c) {
      if (c > 0) {
        if (!tail) {
          load_v(c);
        } else if (wave == 0) {          // the prefetched tail page, zeros after it
#pragma unroll
          for (int q = 0; q < VPL; ++q) vr[q] = q < VT_Q ? vtl[q < VT_Q ? q : 0] : u4{0u, 0u, 0u, 0u};
        }
      }
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {              // the wave's two 32-key blocks
        const int kbase = c * KC + (KC / NWAVE) * wave + 32 * kh;   // relative to k0
        if (kbase >= nk) continue;                   // uniform in the wave
        // V rows kbase + r (r < 32) into the tile: load QPB * kh + q holds row KPW * q + lane / LPK
        constexpr int QPB = 32 / KPW;
#pragma unroll
        for (int q = 0; q < QPB; ++q) {
          const int r = KPW * q + lane / LPK;
          *reinterpret_cast<u4*>(vt + r * VRS + 4 * li) = vr[QPB * kh + q];
        }
        // the tile is written as 16-byte vectors and read as 16-bit halves: keep the compiler from
        // moving either across the other (the wave's own LDS accesses execute in order)
        asm volatile("" ::: "memory");
        // A operand: P rows, keys kbase + 8 grp .. + 7
        bf8 pa;
        {
          const f4 x0 = *reinterpret_cast<const f4*>(prow + kbase + 8 * grp);
          const f4 x1 = *reinterpret_cast<const f4*>(prow + kbase + 8 * grp + 4);
          const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
          uint32_t w[4];
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            uint32_t a = f2bf(x[2 * m]), c2 = f2bf(x[2 * m + 1]);
            if (plo) { a = f2bf(x[2 * m] - bf1((uint16_t)a)); c2 = f2bf(x[2 * m + 1] - bf1((uint16_t)c2)); }
            w[m] = pvalid ? (a | (c2 << 16)) : 0u;
          }
          pa = __builtin_bit_cast(bf8, u4{w[0], w[1], w[2], w[3]});
        }
        // B operands: tile rows 8 grp .. + 7 of dimension 16 cb + col, by LDS transpose reads. In
        // each group of 16 lanes the lanes' 8-byte addresses form a 4 x 16 block of 16-bit values
        // and lane i receives column i of it: lane j supplies tile row 8 grp + j / 4 (+ 4 for the
        // second read) at dimensions 16 cb + 4 (j % 4) .. + 3, so lane col receives the four
        // consecutive keys of dimension 16 cb + col.
        const uint16_t* vt16 = reinterpret_cast<const uint16_t*>(vt);
        const int trow = 8 * grp + (col >> 2), tdim = 4 * (col & 3);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const v4s r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lv4s*)(vt16 + trow * (2 * VRS) + 16 * cb + tdim));
          const v4s r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lv4s*)(vt16 + (trow + 4) * (2 * VRS) + 16 * cb + tdim));
          const u4 w = {(uint32_t)(uint16_t)r0.x | ((uint32_t)(uint16_t)r0.y << 16),
                        (uint32_t)(uint16_t)r0.z | ((uint32_t)(uint16_t)r0.w << 16),
                        (uint32_t)(uint16_t)r1.x | ((uint32_t)(uint16_t)r1.y << 16),
                        (uint32_t)(uint16_t)r1.z | ((uint32_t)(uint16_t)r1.w << 16)};
          oacc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, __builtin_bit_cast(bf8, w), oacc[cb], 0, 0, 0);
        }
        asm volatile("" ::: "memory");
      }
    }
  }
  MARK(3);
  // rows 4a..4a+3 of a lane's accumulators: high and low parts of heads 2a, 2a+1 -> add them; the
  // new key's value row joins in wave 0
  __syncthreads();                       // every wave is done with its V tile (obuf aliases them)
  if (2 * grp < HPG) {
    const float pn0 = last ? sbuf[(2 * grp) * PS + nk] : 0.f, pn1 = last ? sbuf[(2 * grp + 1) * PS + nk] : 0.f;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int d = 16 * cb + col;
      float o0 = oacc[cb][0] + oacc[cb][2], o1 = oacc[cb][1] + oacc[cb][3];
      if (last && wave == 0) {
        o0 = __builtin_fmaf(pn0, vnew[d], o0);
        o1 = __builtin_fmaf(pn1, vnew[d], o1);
      }
      obuf[(wave * HPG + 2 * grp) * D + d] = o0;
      obuf[(wave * HPG + 2 * grp + 1) * D + d] = o1;
    }
  }
  __syncthreads();
  // partial of this split: m[HPG], l[HPG], o[HPG][D] (unnormalised)
  const size_t part = ((size_t)l * p.parts_per_layer + pbase + s_idx) * S::PART;
  const __amdgpu_buffer_rsrc_t Pw = rsrc(p.apart + part);
  static_assert((HPG * D) % 4 == 0, "");
  for (int i = 4 * tx; i < HPG * D; i += 4 * NT) {      // four outputs per thread, waves summed in order
    f4 v = {0.f, 0.f, 0.f, 0.f};
    for (int w = 0; w < NWAVE; ++w) {
      const f4 o = *reinterpret_cast<const f4*>(obuf + w * HPG * D + i);
      v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
    }
    stc4(Pw, 4u * (2 * HPG + i), v);
  }
  if (tx < 2 * HPG) stc(Pw, 4u * tx, ml[tx]);
  MARK(4);
  drain_t(p);
  MARK(5);
  signal(p, ctl, T.sig, false);
  return true;
}

// One slice of the attention output of (sequence b, KV group g): combine the nsplit partials in
// split order (log-sum-exp, P3 "Key Technologies and Architecture": split-KV attention). Each
// (b, g) has `slices` merge tasks over consecutive output ranges, so that the partials are read
// by several CUs at once; one output per thread, MB partials per round trip.
template <class S>
__device__ __forceinline__ bool op_merge(int task) {
  CParams& p = P();
  Ctl& ctl = ctl_s;
  float* sm = smem;
  const TaskHdr T = read_task(p, task);
  constexpr int D = S::D, HPG = S::HPG, MB = 64;
  const int l = T.layer, b = T.a0, g = T.a1, q = T.a2, slices = T.a3, pbase = T.a4, nsplit = T.a5;
  const int tx = tid(), lane = tx & 63, wave = __builtin_amdgcn_readfirstlane(tx >> 6);
  const int ops = (HPG * D) / slices;             // outputs of this slice
  const int nh = ops / D;                         // heads of this slice (a slice is whole heads)
  if (slices < 1 || ops * slices != HPG * D || ops % D != 0 || ops > NT || nh > 2 * NWAVE || nsplit > MERGE_MAX) {
    if (tx == 0) raise_error(p, DEV_STALE, T.id, -1, (uint32_t)slices, (uint32_t)nsplit, (uint32_t)b);
    return false;
  }
  const int o0 = q * ops, h0 = o0 / D;            // first output and first head of the slice
  const __amdgpu_buffer_rsrc_t P0 = rsrc(p.apart + ((size_t)l * p.parts_per_layer + pbase) * S::PART);
  // [2 nh][MERGE_MAX]: per head, m (then the scale) of every split, then l of every split (one head's
  // splits contiguous, so that the combine reads its scales as 16-byte vectors)
  constexpr int SST = MERGE_MAX;
  float* msl = sm;
  float* linv = sm + MERGE_MAX * 2 * 2 * NWAVE;   // [nh] sum over splits of l * scale
  if (!wait_ge(p, ctl, T.w0, (uint32_t)T.t0, T.id)) return false;   // every split of (b, g)
  const bool mine = tx < ops;
  const int o = o0 + tx, hh = tx / D;             // this thread's output and its head in the slice
  float ob[MB];
#pragma unroll
  for (int u = 0; u < MB; ++u) ob[u] = (mine && u < nsplit) ? ldc(P0, 4u * (u * S::PART + 2 * HPG + o)) : 0.f;
  for (int i = tx; i < nsplit * 2 * nh; i += NT) {
    const int s2 = i / (2 * nh), j = i % (2 * nh);
    msl[j * SST + s2] = ldc(P0, 4u * (s2 * S::PART + (j < nh ? h0 + j : HPG + h0 + j - nh)));
  }
  __syncthreads();
  MARK(0);
  // per head: M = max over splits of m, scale_s = exp(m_s - M), L = sum_s l_s scale_s; half a
  // wave per head, lanes over splits
  {
    const int h = 2 * wave + (lane >> 5), sl = lane & 31;
    float M = -INFINITY;
    if (h < nh)
      for (int s2 = sl; s2 < nsplit; s2 += 32) M = fmaxf(M, msl[h * SST + s2]);
    M = wmax<32>(M);
    float Lsum = 0.f;
    if (h < nh)
      for (int s2 = sl; s2 < nsplit; s2 += 32) {
        const float ms = msl[h * SST + s2];
        const float sc = ms == -INFINITY ? 0.f : expf(ms - M);
        msl[h * SST + s2] = sc;
        Lsum = __builtin_fmaf(msl[(nh + h) * SST + s2], sc, Lsum);
      }
    Lsum = wsum<32>(Lsum);
    if (h < nh && sl == 0) linv[h] = Lsum;
  }
  __syncthreads();
  MARK(1);
  if (mine) {
    float acc = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += MB) {
      if (s0 > 0) {
#pragma unroll
        for (int u = 0; u < MB; ++u) ob[u] = (s0 + u < nsplit) ? ldc(P0, 4u * ((s0 + u) * S::PART + 2 * HPG + o)) : 0.f;
      }
      float sc[MB];                      // all scales first (16-byte LDS reads), then the sum
#pragma unroll
      for (int u4 = 0; u4 < MB / 4; ++u4) {
        const f4 v = *reinterpret_cast<const f4*>(msl + hh * SST + s0 + 4 * u4);
#pragma unroll
        for (int c = 0; c < 4; ++c) sc[4 * u4 + c] = s0 + 4 * u4 + c < nsplit ? v[c] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < MB; ++u) acc = __builtin_fmaf(ob[u], sc[u], acc);
    }
    const __amdgpu_buffer_rsrc_t A = rsrc(p.attn + ((size_t)l * MAXB + b) * S::AD + g * HPG * D);
    stc(A, 4u * o, acc / linv[hh]);
  }
  MARK(2);
  drain_t(p);
  MARK(3);
  signal<S::HKV>(p, ctl, T.sig, false, g);   // on KV group g's sub-counters of the attention counter
  return true;
}


// Counter c's signals come in n groups, group g adding to sub-counters g * (CTR_SUB / n) .. (the
// attention merges of KV group g). Wait until the groups' counts reach `target` each for a longer
// leading run of groups than `have` (one poll reads the CTR_SUB lines: one load per lane of wave 0,
// one round trip): returns the number of leading complete groups (> have), or -1 if the step was
// aborted or the watchdog fired.
__device__ int wait_prefix(CParams& p, Ctl& ctl, int c, int n, uint32_t target, int have, int task) {
  const int tx = tid(), lane = tx & 63;
  if (__builtin_amdgcn_readfirstlane(tx >> 6) == 0) {
    int k = -1;
    const uint64_t t0 = now();
    uint32_t it = 0;
    const int per = CTR_SUB / n;
    for (;;) {
      const uint32_t v = lane < CTR_SUB ? ctr_load(ctr_at(p, c, lane)) : 0u;
      int run = 0;
      for (int g = 0; g < n; ++g) {
        uint32_t sum = 0;
        for (int i = 0; i < per; ++i) sum += __builtin_amdgcn_readlane(v, g * per + i);
        if (sum < target) break;
        run = g + 1;
      }
      if (run > have) { k = run; break; }
      __builtin_amdgcn_s_sleep(1);
      if ((++it & 15u) == 0) {
        if (__builtin_amdgcn_readfirstlane(ctr_load(&p.err->abort_flag))) break;
        if (now() - t0 > p.watchdog_ticks) {
          if (lane == 0) raise_error(p, DEV_TIMEOUT, task, c, target, 0, (uint32_t)have);
          break;
        }
      }
    }
    if (lane == 0) {
      ctl.flag = k;
      ctl.t_ready = now();
    }
  }
  __syncthreads();
  const int k = ctl.flag;
  __syncthreads();
  return k;
}

// O projection of one token's attention vector (rows of W_o already in W), one KV group as soon as it
// lands (the ablation flag MK_FLAG_OPROJ_PER_GROUP; P1 "One persistent kernel for the whole decode
// step": the O projection starts when its KV group's attention has landed). Counter c counts every
// merge of the layer, KV group g's on its own sub-counters (wait_prefix), `target` each. Each round
// polls every group in one round trip, stages the columns of every newly complete leading group into
// a_s in one pass and folds their products into the running sums. A lane's 16-byte chunks of a row
// lie in non-decreasing group order and groups are taken in order, so every row's products are summed
// in the order of one pass over the whole row: the same bits as the default form, which waits for
// every group first (measured faster on MI355X, where the four groups' merges land within about a
// microsecond of each other and each extra round adds a dependent staging round trip).
template <class S, int NP, int OT, class Emit>
__device__ __forceinline__ bool oproj_grouped(CParams& p, Ctl& ctl, const WBuf<S::kw(S::AD), NP, S::WF>& W, int nrows, int b0, int nt,
                                              int cbase, int target, bool wait, bool per_group, int task, float* a_s,
                                              __amdgpu_buffer_rsrc_t At, Emit emit) {
  constexpr int AD = S::AD, GW = S::HPG * S::D, HKV = S::HKV;
  static_assert(!S::WF, "the per-KV-group O projection (an ablation) exists for bf16 matrices only");
  using G = Geo<S::kw(AD)>;
  constexpr int NI = (OT * AD + 4 * NT - 1) / (4 * NT);
  static_assert(GW % 4 == 0 && HKV <= 64, "");
  const int tx = tid(), lane = tx & 63, wave = __builtin_amdgcn_readfirstlane(tx >> 6);
  const int lir = lane % G::LPR, rip = lane / G::LPR;
  float acc[NP][OT];
#pragma unroll
  for (int i = 0; i < NP; ++i)
#pragma unroll
    for (int t = 0; t < OT; ++t) acc[i][t] = 0.f;
  int have = 0;
  while (have < HKV) {
    const int k = wait ? wait_prefix(p, ctl, cbase, HKV, (uint32_t)target, per_group ? have : HKV - 1, task) : HKV;
    if (k < 0) return false;
    // columns [have GW, k GW) of every listed token: all loads first, then the LDS writes
    const int w = (k - have) * GW, c0 = have * GW;
    f4 v[NI];
#pragma unroll
    for (int u = 0; u < NI; ++u) {
      const int idx = (u * NT + tx) * 4, t = idx / AD, e = idx - t * AD;
      v[u] = (t < nt && e < w) ? ldc4(At, 4u * ((b0 + t) * AD + c0 + e)) : f4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < NI; ++u) {
      const int idx = (u * NT + tx) * 4, t = idx / AD, e = idx - t * AD;
      if (t < nt && e < w) *reinterpret_cast<f4*>(a_s + t * AD + c0 + e) = v[u];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < G::CPL; ++j) {
      const int e0 = 8 * (lir + G::LPR * j);              // first column of the lane's chunk j
      const int g = e0 / GW;
      if (g < have || g >= k) continue;
#pragma unroll
      for (int t = 0; t < OT; ++t) {
        if (t < nt) {
          const f4* ap = reinterpret_cast<const f4*>(a_s + t * AD + e0);
          const f4 a0 = ap[0], a1 = ap[1];
#pragma unroll
          for (int i = 0; i < NP; ++i) acc[i][t] = dot8(W.w[i][j], a0, a1, acc[i][t]);
        }
      }
    }
    have = k;
  }
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int r = (i * NWAVE + wave) * G::RPP + rip;
#pragma unroll
    for (int t = 0; t < OT; ++t) {
      if (t < nt) {
        const float s = wsum<G::LPR>(acc[i][t]);
        if (lir == 0 && r < nrows) emit(r, t, s);
      }
    }
  }
  return true;
}

// Output rows row0..row0+nrows of the layer for every token: the fused residual add that rejoins
// both branches (P1 "One persistent kernel for the whole decode step"):
//   x_{l+1} = (x_l + W_o attn) + sum_i w_i W_down[e_i] h_i   (experts in ascending index).
// Waits for the routing table (to prefetch the right W_down rows), then for the MoE slices (the
// MoE term is formed first), then for the attention of every KV group.
template <class S, int TB, int VAR>
__device__ __forceinline__ bool op_out(int task) {
  CParams& p = P();
  Ctl& ctl = ctl_s;
  float* sm = smem;
  const TaskHdr T = read_task(p, task);
  constexpr int H = S::H, AD = S::AD, F = S::F, K = S::K;
  constexpr int NPO = (OUT_MAXR + NWAVE * Geo<S::kw(AD)>::RPP - 1) / (NWAVE * Geo<S::kw(AD)>::RPP);
  constexpr int NPD = (OUT_MAXR * K + NWAVE * Geo<S::kw(F)>::RPP - 1) / (NWAVE * Geo<S::kw(F)>::RPP);
  const int l = T.layer, row0 = T.a0, nrows = T.a1;
  const auto& Lp = cst(p.layers)[l];
  auto orow = [&](int r) { return Lp.w_o + (size_t)(row0 + r) * S::rw(AD); };
  WBuf<S::kw(AD), NPO, S::WF> WO;
  const bool pre = !(p.flags & 2);
  if (pre) load_block<S::kw(AD), NPO, S::WF>(WO, 0, nrows, orow);
  if (!wait_ge(p, ctl, T.w0, (uint32_t)T.t0, T.id)) return false;      // routing known
  load_route(p, l);
  const RouteTable& rt = ctl.rt;
  float* a_s = sm;                                                     // [AD]
  float* h_s = sm + AD;                                                // [K][F]
  float* o_s = h_s + K * F;                                            // [OUT_MAXR]
  float* y_s = o_s + OUT_MAXR;                                         // [K][OUT_MAXR]
  if (!pre) load_block<S::kw(AD), NPO, S::WF>(WO, 0, nrows, orow);
  float* mo_s = y_s + K * OUT_MAXR;                                    // [MAXB][OUT_MAXR] MoE term
  float* xv_s = mo_s + MAXB * OUT_MAXR;                                // [MAXB][OUT_MAXR] x_l rows
  const __amdgpu_buffer_rsrc_t Hb = rsrc(p.h + (size_t)l * MAXB * K * F);
  const __amdgpu_buffer_rsrc_t At = rsrc(p.attn + (size_t)l * MAXB * AD);
  const __amdgpu_buffer_rsrc_t Xn = rsrc(p.x + (size_t)(l + 1) * MAXB * H);
  // MoE branch first: the expert slices finish before the attention merges, so only the O
  // projection and the residual add remain once attention is in
  for (int b = 0; b < p.B; ++b) {
    int sel[K];
#pragma unroll
    for (int i = 0; i < K; ++i) sel[i] = rt.sel[b][i];
    auto drow = [&](int q) {   // q = i * nrows + r
      const int i = q / nrows, r = q % nrows;
      int e = 0;
#pragma unroll
      for (int ii = 0; ii < K; ++ii) if (ii == i) e = sel[ii];
      return Lp.w_down + ((size_t)e * H + row0 + r) * S::rw(F);
    };
    WBuf<S::kw(F), NPD, S::WF> WD;
    load_block<S::kw(F), NPD, S::WF>(WD, 0, K * nrows, drow);
    if (b == 0 && !wait_ge(p, ctl, T.w1, (uint32_t)T.t1, T.id)) return false;   // every MoE slice
    stage_f4<K * F>(h_s, Hb, 4u * (b * K * F), K * F);
    __syncthreads();
    if (b == 0) MARK(0);
    compute_block<S::kw(F), NPD, 1, S::WF>(WD, 0, K * nrows, 1, [&](int q, int t) { return h_s + (q / nrows) * F; },
                             [&](int q, int t, float v) { y_s[(q / nrows) * OUT_MAXR + q % nrows] = v; });
    __syncthreads();
    if (tid() < nrows) {
      const int r = tid(), row = row0 + r;
      float xv;
      if (l == 0) {
        int tok = cst(p.tokens)[b];
        tok = (tok < 0 || tok >= p.V) ? 0 : tok;
        xv = bf1(p.embed[(size_t)tok * H + row]);
      } else {
        xv = ldc(rsrc(p.x + ((size_t)l * MAXB + b) * H), 4u * row);
      }
      float moe = 0.f;
      for (int i = 0; i < K; ++i)
        moe = moe + rt.w[b][i] * y_s[i * OUT_MAXR + r];
      mo_s[b * OUT_MAXR + r] = moe;
      xv_s[b * OUT_MAXR + r] = xv;
    }
  }
  MARK(1);
  // the per-KV-group form is compiled into a kernel instance of its own (VAR 1), so that its code does
  // not change the register allocation of the default form
  constexpr bool per_group = VAR == 1;
  if (!per_group && !wait_ge(p, ctl, T.a2, (uint32_t)T.a3, T.id)) return false;   // attention of every KV group
  for (int b = 0; b < p.B; ++b) {
    if constexpr (per_group) {      // KV group by KV group as each group's merges land (ablation)
      if (!oproj_grouped<S, NPO, 1>(p, ctl, WO, nrows, b, 1, T.a2, T.a3 / S::HKV, b == 0, true, T.id, a_s, At,
                                    [&](int r, int t, float v) { o_s[r] = v; }))
        return false;
    } else {
      stage_f4<AD>(a_s, At, 4u * (b * AD), AD);
      __syncthreads();
      compute_block_shared<S::kw(AD), NPO, 1, 1, S::WF>(WO, 0, nrows, 1, [&](int r, int t) { return a_s; },
                                       [&](int r, int t, float v) { o_s[r] = v; });
    }
    if (b == 0) MARK(2);
    __syncthreads();
    if (tid() < nrows) {
      const int r = tid(), row = row0 + r;
      const float xn = (xv_s[b * OUT_MAXR + r] + o_s[r]) + mo_s[b * OUT_MAXR + r];
      stc(Xn, 4u * (b * H + row), xn);
      if (p.hidden_out && l == p.L - 1) p.hidden_out[(size_t)b * H + row] = xn;
    }
    __syncthreads();
  }
  MARK(3);
  drain_t(p);
  MARK(4);
  signal(p, ctl, T.sig, false);
  return true;
}

// Output rows for a batch of several tokens: the same sums as op_out, in the same order (so the
// results are bitwise those of the one-token form), laid out for latency:
//   * the x_l rows of every token are requested once, up front;
//   * the MoE term is pipelined over tokens: the W_down rows and the h vectors of token b+1 are in
//     flight while token b is multiplied (two register buffers, two LDS h buffers);
//   * the attention vectors of OT tokens are staged together and the O projection multiplies them
//     in one pass over the W_o rows.
template <class S, int TB>
__device__ __forceinline__ bool op_out_batch(int task) {
  CParams& p = P();
  Ctl& ctl = ctl_s;
  float* sm = smem;
  const TaskHdr T = read_task(p, task);
  constexpr int H = S::H, AD = S::AD, F = S::F, K = S::K, KF = K * F;
  using LY = OutLds<S>;
  constexpr int NPO = (OUT_MAXR + NWAVE * Geo<S::kw(AD)>::RPP - 1) / (NWAVE * Geo<S::kw(AD)>::RPP);
  constexpr int NPD = (OUT_MAXR * K + NWAVE * Geo<S::kw(F)>::RPP - 1) / (NWAVE * Geo<S::kw(F)>::RPP);
  constexpr int HI = (KF + 4 * NT - 1) / (4 * NT);
  const int l = T.layer, row0 = T.a0, nrows = T.a1, B = p.B;
  const auto& Lp = cst(p.layers)[l];
  float* y_s = sm + LY::Y;
  float* mo_s = sm + LY::MO;
  float* xv_s = sm + LY::XV;
  float* o_s = sm + LY::O;
  if (!wait_ge(p, ctl, T.w0, (uint32_t)T.t0, T.id)) return false;      // routing known
  load_route(p, l);
  const RouteTable& rt = ctl.rt;
  const __amdgpu_buffer_rsrc_t Hb = rsrc(p.h + (size_t)l * MAXB * K * F);
  const __amdgpu_buffer_rsrc_t At = rsrc(p.attn + (size_t)l * MAXB * AD);
  const __amdgpu_buffer_rsrc_t Xn = rsrc(p.x + (size_t)(l + 1) * MAXB * H);
  // x_l[b][row0 + r] for every (b, r): one value per thread, written to LDS after the MoE term
  float xv = 0.f;
  const int tx = tid();
  if (tx < B * nrows) {
    const int b = tx / nrows, row = row0 + tx % nrows;
    if (l == 0) {
      int tok = cst(p.tokens)[b];
      tok = (tok < 0 || tok >= p.V) ? 0 : tok;
      xv = bf1(p.embed[(size_t)tok * H + row]);
    } else {
      xv = ldc(rsrc(p.x + ((size_t)l * MAXB + b) * H), 4u * row);
    }
  }
  if (T.a4 & 4) {
    // the O projection and the down projections were computed by queued items (o[l][b][row] and
    // y[b][i][row]): x_l+1 = (x_l + o) + MoE term, the MoE term in ascending expert order - the same
    // sums in the same order as the form below
    if (!wait_ge(p, ctl, T.w1, (uint32_t)T.t1, T.id)) return false;   // every expert task (all items)
    MARK(0);
    if (tx < B * nrows) {
      const int b = tx / nrows, r = tx % nrows, row = row0 + r;
      const __amdgpu_buffer_rsrc_t Yr = rsrc(p.y + (size_t)l * MAXB * K * H);
      const __amdgpu_buffer_rsrc_t Ob = rsrc(p.o + (size_t)l * MAXB * H);
      float yv[K];
#pragma unroll
      for (int i = 0; i < K; ++i) yv[i] = ldc(Yr, 4u * ((b * K + i) * H + row));
      const float ov = ldc(Ob, 4u * (b * H + row));
      float moe = 0.f;
#pragma unroll
      for (int i = 0; i < K; ++i) moe = moe + rt.w[b][i] * yv[i];
      const float xn = (xv + ov) + moe;
      stc(Xn, 4u * (b * H + row), xn);
      if (p.hidden_out && l == p.L - 1) p.hidden_out[(size_t)b * H + row] = xn;
    }
    MARK(3);
    drain_t(p);
    signal(p, ctl, T.sig, false);
    return true;
  }
  if (T.a4) {
    // the down projections were computed by the queued down items: y[b][i][row] for token b's i-th
    // expert; the MoE term sums w_i y_i in ascending expert order, as the form below does
    WBuf<S::kw(AD), NPO, S::WF> WO;
    auto orow = [&](int r) { return Lp.w_o + (size_t)(row0 + r) * S::rw(AD); };
    load_block<S::kw(AD), NPO, S::WF>(WO, 0, nrows, orow);
    if (!wait_ge(p, ctl, T.w1, (uint32_t)T.t1, T.id)) return false;   // every expert task (all items)
    MARK(0);
    if (tx < B * nrows) {
      const int b = tx / nrows, r = tx % nrows;
      const __amdgpu_buffer_rsrc_t Yr = rsrc(p.y + (size_t)l * MAXB * K * H);
      float yv[K];
#pragma unroll
      for (int i = 0; i < K; ++i) yv[i] = ldc(Yr, 4u * ((b * K + i) * H + row0 + r));
      float moe = 0.f;
#pragma unroll
      for (int i = 0; i < K; ++i) moe = moe + rt.w[b][i] * yv[i];
      mo_s[b * OUT_MAXR + r] = moe;
      xv_s[b * OUT_MAXR + r] = xv;
    }
    MARK(1);
    float* a_s = sm + LY::A;
    if (!wait_ge(p, ctl, T.a2, (uint32_t)T.a3, T.id)) return false;      // attention of every KV group
    for (int b0 = 0; b0 < B; b0 += OUT_OT) {
      const int nt = B - b0 < OUT_OT ? B - b0 : OUT_OT;
      stage_f4<OUT_OT * AD>(a_s, At, 4u * (b0 * AD), nt * AD);
      __syncthreads();
      if (b0 == 0) MARK(2);
      compute_block_shared<S::kw(AD), NPO, OUT_OT, TG_ROWS<S>, S::WF>(WO, 0, nrows, nt, [&](int r, int t) { return a_s + t * AD; },
                                            [&](int r, int t, float v) { o_s[t * OUT_MAXR + r] = v; });
      __syncthreads();
      if (tx < nt * nrows) {
        const int t = tx / nrows, r = tx % nrows, b = b0 + t, row = row0 + r;
        const float xn = (xv_s[b * OUT_MAXR + r] + o_s[t * OUT_MAXR + r]) + mo_s[b * OUT_MAXR + r];
        stc(Xn, 4u * (b * H + row), xn);
        if (p.hidden_out && l == p.L - 1) p.hidden_out[(size_t)b * H + row] = xn;
      }
      __syncthreads();
    }
    MARK(3);
    drain_t(p);
    MARK(4);
    signal(p, ctl, T.sig, false);
    return true;
  }
  // W_down rows of token b: q = i * nrows + r is row row0 + r of its i-th expert
  auto drow_of = [&](int b) {
    return [&, b](int q) {
      const int i = q / nrows, r = q - i * nrows;
      return Lp.w_down + ((size_t)rt.sel[b][i] * H + row0 + r) * S::rw(F);
    };
  };
  f4 hv[HI];
  auto h_issue = [&](int b) {
#pragma unroll
    for (int u = 0; u < HI; ++u) {
      const int i = (u * NT + tx) * 4;
      hv[u] = i < KF ? ldc4(Hb, 4u * (b * KF + i)) : f4{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto h_put = [&](float* dst) {
#pragma unroll
    for (int u = 0; u < HI; ++u) {
      const int i = (u * NT + tx) * 4;
      if (i < KF) *reinterpret_cast<f4*>(dst + i) = hv[u];
    }
  };
  // token b's MoE term from its W_down rows (in W) and its h (staged at hs)
  auto moe_token = [&](const WBuf<S::kw(F), NPD, S::WF>& W, const float* hs, int b) {
    compute_block<S::kw(F), NPD, 1, S::WF>(W, 0, K * nrows, 1, [&](int q, int t) { return hs + (q / nrows) * F; },
                             [&](int q, int t, float v) { y_s[(q / nrows) * OUT_MAXR + q % nrows] = v; });
    __syncthreads();
    if (tx < nrows) {
      float moe = 0.f;
      for (int i = 0; i < K; ++i) moe = moe + rt.w[b][i] * y_s[i * OUT_MAXR + tx];
      mo_s[b * OUT_MAXR + tx] = moe;
    }
  };
  float* hA = sm + LY::HA;
  float* hB = sm + LY::HB;
  WBuf<S::kw(F), NPD, S::WF> WA, WB;
  load_block<S::kw(F), NPD, S::WF>(WA, 0, K * nrows, drow_of(0));
  if (!wait_ge(p, ctl, T.w1, (uint32_t)T.t1, T.id)) return false;   // every MoE slice
  h_issue(0);
  h_put(hA);
  MARK(0);
  for (int b = 0; b < B; b += 2) {
    const bool has1 = b + 1 < B;
    if (has1) { load_block<S::kw(F), NPD, S::WF>(WB, 0, K * nrows, drow_of(b + 1)); h_issue(b + 1); }
    __syncthreads();                       // hA staged; the previous token is done with y_s
    moe_token(WA, hA, b);
    if (has1) h_put(hB);
    if (b + 2 < B) { load_block<S::kw(F), NPD, S::WF>(WA, 0, K * nrows, drow_of(b + 2)); h_issue(b + 2); }
    if (has1) {
      __syncthreads();                     // hB staged; token b is done with y_s and hA
      moe_token(WB, hB, b + 1);
      if (b + 2 < B) h_put(hA);
    }
  }
  if (tx < B * nrows) xv_s[(tx / nrows) * OUT_MAXR + tx % nrows] = xv;
  MARK(1);
  // O projection of OUT_OT tokens per pass over the W_o rows
  auto orow = [&](int r) { return Lp.w_o + (size_t)(row0 + r) * S::rw(AD); };
  WBuf<S::kw(AD), NPO, S::WF> WO;
  load_block<S::kw(AD), NPO, S::WF>(WO, 0, nrows, orow);
  __syncthreads();                         // the MoE phase is done with the LDS it shares with a_s
  float* a_s = sm + LY::A;
  if (!wait_ge(p, ctl, T.a2, (uint32_t)T.a3, T.id)) return false;      // attention of every KV group
  for (int b0 = 0; b0 < B; b0 += OUT_OT) {
    const int nt = B - b0 < OUT_OT ? B - b0 : OUT_OT;
    stage_f4<OUT_OT * AD>(a_s, At, 4u * (b0 * AD), nt * AD);
    __syncthreads();
    if (b0 == 0) MARK(2);
    compute_block_shared<S::kw(AD), NPO, OUT_OT, TG_ROWS<S>, S::WF>(WO, 0, nrows, nt, [&](int r, int t) { return a_s + t * AD; },
                                          [&](int r, int t, float v) { o_s[t * OUT_MAXR + r] = v; });
    __syncthreads();
    if (tx < nt * nrows) {
      const int t = tx / nrows, r = tx % nrows, b = b0 + t, row = row0 + r;
      const float xn = (xv_s[b * OUT_MAXR + r] + o_s[t * OUT_MAXR + r]) + mo_s[b * OUT_MAXR + r];
      stc(Xn, 4u * (b * H + row), xn);
      if (p.hidden_out && l == p.L - 1) p.hidden_out[(size_t)b * H + row] = xn;
    }
    __syncthreads();
  }
  MARK(3);
  drain_t(p);
  MARK(4);
  signal(p, ctl, T.sig, false);
  return true;
}

// lm_head rows row0..row0+nrows: logits = W_lm . RMSNorm_final(x_L), plus the running greedy
// argmax (first index of the maximum) through a 64-bit atomic max on (ordered logit, ~index).
template <class S, int TB>
__device__ __forceinline__ bool op_lmhead(int task) {
  CParams& p = P();
  Ctl& ctl = ctl_s;
  float* sm = smem;
  const TaskHdr T = read_task(p, task);
  // several tokens: more row passes per block, so that each activation read from LDS serves more rows
  constexpr int H = S::H, KW = S::kw(H), NP = (Geo<KW>::CPL >= 4) ? (TB > 1 ? 4 : 2) : 4, RPP = Geo<KW>::RPP;
  const int row0 = T.a0, nrows = T.a1;
  auto rowptr = [&](int r) { return p.lm_head + (size_t)(row0 + r) * S::rw(H); };
  const bool pre = !(p.flags & 2);
  float* logits = p.logits;
  const int V = p.V;
  const int tx = tid(), lane = tx & 63, wave = __builtin_amdgcn_readfirstlane(tx >> 6);
  // the running greedy argmax key of token t (first index of the maximum) into p.amax[t]
  auto publish = [&](int t, float best, int besti) {
    if (besti != 0x7fffffff) {
      uint32_t u = __float_as_uint(best);
      u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
      const unsigned long long key = ((unsigned long long)u << 32) | (0xffffffffu - (uint32_t)besti);
      __hip_atomic_fetch_max(p.amax + t, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  if constexpr (TB > 1) {                        // several tokens: the matrix cores
    MRows<S> A;
    if (pre) mrows_load<S>(A, 0, nrows, rowptr);
    if (!wait_ge(p, ctl, T.w0, (uint32_t)T.t0, T.id)) return false;
    if (tid() < MAXB) ctl.toks[tid()] = tid();
    __syncthreads();
    stage_norm<S, MRows<S>::AS>(p, p.L, ctl.toks, p.B, p.final_norm, sm, T.id);
    // thread 8 i + t sees rows i, i + 16, ... of token t, in ascending order
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    auto em = [&](int r, int t, float v) {
      const int row = row0 + r;
      if (logits) __builtin_nontemporal_store(v, logits + (size_t)t * V + row);
      if (v > bv || (v == bv && row < bi)) { bv = v; bi = row; }
    };
    mrows_stream<S>(A, pre, nrows, p.B, rowptr, sm, sm + MRows<S>::RED, em);
    float* cv = sm + MRows<S>::END;                 // [16][8]
    int* ci = reinterpret_cast<int*>(cv + 128);
    if (tx < 128) { cv[tx] = bv; ci[tx] = bi; }
    __syncthreads();
    if (tx < p.B) {
      float best = -INFINITY;
      int besti = 0x7fffffff;
      for (int i = 0; i < 16; ++i) {
        const float v = cv[8 * i + tx];
        const int ii = ci[8 * i + tx];
        if (v > best || (v == best && ii < besti)) { best = v; besti = ii; }
      }
      publish(tx, best, besti);
    }
  } else {
    WBuf<KW, NP, S::WF> A;
    if (pre) load_block<KW, NP, S::WF>(A, 0, nrows, rowptr);
    if (!wait_ge(p, ctl, T.w0, (uint32_t)T.t0, T.id)) return false;
    if (tid() < MAXB) ctl.toks[tid()] = tid();
    __syncthreads();
    stage_norm<S>(p, p.L, ctl.toks, p.B, p.final_norm, sm, T.id);
    float bv[TB];
    int bi[TB];
#pragma unroll
    for (int t = 0; t < TB; ++t) { bv[t] = -INFINITY; bi[t] = 0x7fffffff; }
    gemv_stream<KW, NP, TB, TG_ROWS<S>, S::WF>(A, pre, nrows, p.B, rowptr,
        [&](int r, int t) { return sm + (size_t)t * H; },
        [&](int r, int t, float v) {
          const int row = row0 + r;
          if (logits) __builtin_nontemporal_store(v, logits + (size_t)t * V + row);
#pragma unroll
          for (int tt = 0; tt < TB; ++tt)
            if (tt == t && (v > bv[tt] || (v == bv[tt] && row < bi[tt]))) { bv[tt] = v; bi[tt] = row; }
        });
    // combine the emitting lanes (lir == 0) of every wave, then one atomic per token
    float* cv = sm + (size_t)TB * H;                                 // [NWAVE * RPP][TB]
    int* ci = reinterpret_cast<int*>(cv + NWAVE * RPP * TB);
    if (lane % Geo<KW>::LPR == 0) {
      const int slot = wave * RPP + lane / Geo<KW>::LPR;
#pragma unroll
      for (int t = 0; t < TB; ++t) { cv[slot * TB + t] = bv[t]; ci[slot * TB + t] = bi[t]; }
    }
    __syncthreads();
    if (tid() < p.B) {
      const int t = tid();
      float best = -INFINITY;
      int besti = 0x7fffffff;
      for (int s = 0; s < NWAVE * RPP; ++s) {
        const float v = cv[s * TB + t];
        const int i = ci[s * TB + t];
        if (v > best || (v == best && i < besti)) { best = v; besti = i; }
      }
      publish(t, best, besti);
    }
  }
  signal(p, ctl, T.sig, false);
  return true;
}

// End of the worker's queue: the last worker to finish publishes the argmax and clears every
// counter and the argmax keys for the next step (single assignment per step: nothing else needs
// clearing).
__device__ void finish(CParams& p, Ctl& ctl) {
  drain();
  __syncthreads();
  // end-of-step detection in two levels: the last worker of each sub-counter of done_ctr bumps
  // the line after the last counter; the last of those resets the counters
  uint32_t* top = p.ctr + (size_t)p.n_ctr * CTR_SUB * CTR_STRIDE;
  if (tid() == 0) {
    const int s = (int)(blockIdx.x % CTR_SUB);
    const uint32_t n_s = (uint32_t)((p.n_workers - s + CTR_SUB - 1) / CTR_SUB);
    const uint32_t nsub = (uint32_t)(p.n_workers < CTR_SUB ? p.n_workers : CTR_SUB);
    int last = 0;
    if (ctr_add(ctr_at(p, p.done_ctr, s), 1u) == n_s - 1) last = ctr_add(top, 1u) == nsub - 1;
    ctl.flag = last;
  }
  __syncthreads();
  if (!ctl.flag) return;
  if (tid() < MAXB) {
    const unsigned long long key = __hip_atomic_load(p.amax + tid(), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (p.argmax_out && tid() < p.B) p.argmax_out[tid()] = (int32_t)(0xffffffffu - (uint32_t)key);
    __hip_atomic_store(p.amax + tid(), 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  for (int i = tid(); i < p.n_ctr * CTR_SUB; i += NT)
    if (i / CTR_SUB != p.done_ctr) __hip_atomic_store(p.ctr + (size_t)i * CTR_STRIDE, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int i = tid(); i < p.L * MAX_SLOTS; i += NT)
    __hip_atomic_store(p.slot_ctr + (size_t)i * CTR_STRIDE, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  drain();
  __syncthreads();
  if (tid() < CTR_SUB) __hip_atomic_store(ctr_at(p, p.done_ctr, tid()), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (tid() == 0) __hip_atomic_store(top, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <class S, int TB, int VAR>
__global__ void __launch_bounds__(NT, 2) mk_step(Params) {
  CParams& p = P();
  const int qs = cst(p.qoff)[blockIdx.x], qe = cst(p.qoff)[blockIdx.x + 1];
  const bool trace = (p.flags & 1) && p.trace;
  {
    // the step's RoPE table: angle in double precision (R3), then rounded to float
    constexpr int D = S::D;
    float* tab = rope_tab<S, TB>();
    for (int i = tid(); i < p.B * (D / 2); i += NT) {
      const int b = i / (D / 2), j = i % (D / 2);
      const double ang = (double)cst(p.positions)[b] * cst(p.inv_freq)[j];
      tab[b * D + j] = (float)cos(ang);
      tab[b * D + D / 2 + j] = (float)sin(ang);
    }
    if (tid() == 0) ctl_s.norm_l = -1;
    __syncthreads();
  }
  for (int ti = qs; ti < qe; ++ti) {
    const int op = cst(p.tasks)[(size_t)ti * DESC_WORDS + D_OP];
    // every other op overwrites the LDS area where expert slices keep the staged normed input
    if (op != OP_GATEUP && tid() == 0) ctl_s.norm_l = -1;
    const uint64_t t_start = trace ? now() : 0;
    if (trace && tid() == 0) {
      ctl_s.t_ready = t_start;
#pragma unroll
      for (int i = 0; i < TRACE_MARKS; ++i) ctl_s.mark[i] = 0;
      ctl_s.mark[7] = __builtin_amdgcn_s_memtime();   // shader clock at the start (cycles over the task)
    }
    if (trace) __syncthreads();
    bool ok;
    switch (op) {
      case OP_QKV: ok = op_qkv<S, TB, VAR>(ti); break;
      case OP_ROUTER: ok = op_router<S, TB>(ti); break;
      case OP_GATEUP: ok = op_gateup<S, TB>(ti); break;
      case OP_ATTN: ok = op_attn<S, TB, VAR>(ti); break;
      case OP_OUT:
        if constexpr (TB == 1) ok = op_out<S, TB, VAR>(ti);
        else ok = op_out_batch<S, TB>(ti);
        break;
      case OP_LMHEAD: ok = op_lmhead<S, TB>(ti); break;
      case OP_MERGE: ok = op_merge<S>(ti); break;
      default:
        if (tid() == 0) raise_error(p, DEV_BAD_OP, ti, -1, 0, (uint32_t)op, 0);
        ok = false;
    }
    if (trace) __syncthreads();          // t_end: every wave is done with the task
    if (trace && tid() == 0) {
      unsigned long long* tr = p.trace + (size_t)ti * TRACE_WORDS;
      tr[0] = (unsigned long long)ti | ((unsigned long long)blockIdx.x << 32);
      tr[1] = t_start;
      tr[2] = ctl_s.t_ready;
      tr[3] = now();
      ctl_s.mark[7] = __builtin_amdgcn_s_memtime() - ctl_s.mark[7];
#pragma unroll
      for (int i = 0; i < TRACE_MARKS; ++i) tr[4 + i] = ctl_s.mark[i];
    }
    if (!ok) break;
    __syncthreads();
  }
  finish(p, ctl_s);
}

// ------------------------------------------------------------------------------ host side

template <class S>
constexpr size_t lds_bytes(int tb) {
  return ((size_t)rope_off<S>(tb) + (size_t)tb * S::D) * 4;   // RoPE table: tb sequences
}
// two workers per CU: both workers' LDS (dynamic + the static control block) within 160 KB
static_assert(2 * (lds_bytes<ShapeFull>(1) + sizeof(Ctl)) <= 160 * 1024, "batch-1 kernel: LDS for two workers per CU");
static_assert(2 * (lds_bytes<ShapeFull>(MAXB) + sizeof(Ctl)) <= 160 * 1024, "batch-8 kernel: LDS for two workers per CU");

template <class S, int TB, int VAR = 0>
static hipError_t launch_one(const Params& p, int grid, hipStream_t st, size_t* lds_out) {
  const size_t lds = lds_bytes<S>(TB);
  if (lds_out) *lds_out = lds;
  hipError_t e = hipFuncSetAttribute((const void*)mk_step<S, TB, VAR>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  Params pp = p;
  void* args[] = {&pp};
  return hipLaunchCooperativeKernel((const void*)mk_step<S, TB, VAR>, dim3(grid), dim3(NT), args, (unsigned)lds, st);
}

template <class S, int TB, int VAR = 0>
static hipError_t occupancy_one(int* blocks_per_cu) {
  const size_t lds = lds_bytes<S>(TB);
  hipError_t e = hipFuncSetAttribute((const void*)mk_step<S, TB, VAR>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, (const void*)mk_step<S, TB, VAR>, NT, lds);
}

// 0 / 1: the small and the full shape with bf16 matrices; 2 / 3: the same with FP8 matrices; 4 / 5:
// with MXFP4 matrices
int shape_id(int H, int D, int HQ, int HKV, int E, int K, int F, int wf) {
  int id = -1;
  if (H == ShapeSmall::H && D == ShapeSmall::D && HQ == ShapeSmall::HQ && HKV == ShapeSmall::HKV &&
      E == ShapeSmall::E && K == ShapeSmall::K && F == ShapeSmall::F) id = 0;
  if (H == ShapeFull::H && D == ShapeFull::D && HQ == ShapeFull::HQ && HKV == ShapeFull::HKV &&
      E == ShapeFull::E && K == ShapeFull::K && F == ShapeFull::F) id = 1;
  return id < 0 || wf < 0 || wf > 2 ? -1 : id + 2 * wf;
}

// Kernel instances: batch 1 (VAR 1: the per-KV-group O projection of MK_FLAG_OPROJ_PER_GROUP) and
// batch > 1 (VAR 2: the QKV tasks publish the step's K/V, for rows of one sequence in one step).
int step_variant(int batch, int flags, bool kv_first) {
  if (batch == 1) return (flags & 8) ? 1 : 0;
  return kv_first ? 2 : 0;
}

// The instance of shape S for (batch, var), run through fn.run<S, TB, VAR>(); VAR 1 exists for bf16
// matrices only
template <class S, class Fn>
static hipError_t with_instance(int batch, int var, const Fn& fn) {
  if (batch > 1) return var == 2 ? fn.template run<S, MAXB, 2>() : fn.template run<S, MAXB, 0>();
  if (var == 1) {
    if constexpr (S::WF == 0) return fn.template run<S, 1, 1>();
    else return hipErrorInvalidValue;
  }
  return fn.template run<S, 1, 0>();
}

template <class Fn>
static hipError_t with_shape(int shape, int batch, int var, const Fn& fn) {
  switch (shape) {
    case 0: return with_instance<ShapeSmall>(batch, var, fn);
    case 1: return with_instance<ShapeFull>(batch, var, fn);
    case 2: return with_instance<ShapeSmall8>(batch, var, fn);
    case 3: return with_instance<ShapeFull8>(batch, var, fn);
    case 4: return with_instance<ShapeSmall4>(batch, var, fn);
    case 5: return with_instance<ShapeFull4>(batch, var, fn);
    default: return hipErrorInvalidValue;
  }
}

struct LaunchFn {
  const Params& p;
  int grid;
  hipStream_t st;
  size_t* lds;
  template <class S, int TB, int VAR>
  hipError_t run() const { return launch_one<S, TB, VAR>(p, grid, st, lds); }
};

struct OccupancyFn {
  int* blocks_per_cu;
  template <class S, int TB, int VAR>
  hipError_t run() const { return occupancy_one<S, TB, VAR>(blocks_per_cu); }
};

hipError_t launch_step(int shape, int batch, int var, const Params& p, int grid, hipStream_t st, size_t* lds) {
  return with_shape(shape, batch, var, LaunchFn{p, grid, st, lds});
}

hipError_t step_occupancy(int shape, int batch, int var, int* blocks_per_cu) {
  return with_shape(shape, batch, var, OccupancyFn{blocks_per_cu});
}

// Plain streaming read of n16 16-byte words (a bandwidth ceiling for comparison with the step
// kernel): four non-temporal loads in flight per thread; the words are folded so the loads stay, and
// the fold is stored only if it equals a constant (never, in practice; `sink` is then a valid word).
__global__ void __launch_bounds__(256) stream_read(const u4* __restrict__ src, size_t n16, uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u4 a = ldw(src + i), b = ldw(src + i + stride), c = ldw(src + i + 2 * stride), d = ldw(src + i + 3 * stride);
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const u4 a = ldw(src + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

hipError_t launch_stream_read(const void* src, size_t n16, uint32_t* sink, int blocks, hipStream_t st) {
  hipLaunchKernelGGL(stream_read, dim3(blocks), dim3(256), 0, st, static_cast<const u4*>(src), n16, sink);
  return hipGetLastError();
}

// Hand-off litmus test of the step kernel's protocol, across every XCD: in round r one workgroup
// (the producer, a different one each round) writes `words` words = r with sc1 stores, waits for
// them (s_waitcnt vmcnt(0)), passes a workgroup barrier and bumps `flag` with one relaxed
// agent-scope atomic add - exactly what a task does before signalling. Every other workgroup polls
// `flag` from wave 0 with relaxed agent-scope loads, passes a barrier and reads the words with sc1
// loads - exactly what a task does after its dependency wait - and counts words that are not r
// (stale). A consumer then bumps `done`; the next producer waits for every consumer of the previous
// round before it overwrites the words. Every wait is bounded by the watchdog (res[3] set, and every
// workgroup leaves its loop once it sees that), so the grid always drains.
// res (uint32 words): [0..1] stale words and [2..3] words checked (64-bit), [4] rounds completed by
// workgroup 0, [5] watchdog fired.
__device__ bool litmus_wait(uint32_t* c, uint32_t target, uint32_t* res, uint64_t wd) {
  __shared__ int ok_s;
  const int tx = tid(), lane = tx & 63;
  if (__builtin_amdgcn_readfirstlane(tx >> 6) == 0) {
    int ok = 1;
    const uint64_t t0 = now();
    uint32_t it = 0;
    while (__builtin_amdgcn_readfirstlane(ctr_load(c)) < target) {
      __builtin_amdgcn_s_sleep(1);
      if ((++it & 15u) == 0) {
        if (__builtin_amdgcn_readfirstlane(ctr_load(res + 5)) != 0u) { ok = 0; break; }
        if (now() - t0 > wd) {
          if (lane == 0) __hip_atomic_store(res + 5, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ok = 0;
          break;
        }
      }
    }
    if (lane == 0) ok_s = ok;
  }
  __syncthreads();
  const bool ok = ok_s != 0;
  __syncthreads();
  return ok;
}

__global__ void __launch_bounds__(NT) handoff_litmus(uint32_t* data, uint32_t* flag, uint32_t* done, uint32_t* res,
                                                     int rounds, int words, uint64_t wd) {
  const int G = (int)gridDim.x, me = (int)blockIdx.x, tx = tid();
  const __amdgpu_buffer_rsrc_t Dt = rsrc(data);
  uint32_t stale = 0, checked = 0;
  int r = 1;
  for (; r <= rounds; ++r) {
    const int prod = (int)(((unsigned)r * 37u + 11u) % (unsigned)G);
    if (me == prod) {
      if (!litmus_wait(done, (uint32_t)(G - 1) * (uint32_t)(r - 1), res, wd)) break;
      for (int i = tx; i < words; i += NT) stci(Dt, 4u * i, r);
      drain();
      __syncthreads();
      if (tx == 0) ctr_add(flag, 1u);
    } else {
      if (!litmus_wait(flag, (uint32_t)r, res, wd)) break;
      for (int i = tx; i < words; i += NT) {
        stale += ldci(Dt, 4u * i) != r ? 1u : 0u;
        ++checked;
      }
      __syncthreads();                 // every thread of the consumer has read the round's words
      if (tx == 0) ctr_add(done, 1u);
    }
  }
  if (stale) atomicAdd(reinterpret_cast<unsigned long long*>(res), (unsigned long long)stale);
  if (checked) atomicAdd(reinterpret_cast<unsigned long long*>(res + 2), (unsigned long long)checked);
  if (me == 0 && tx == 0) atomicAdd(res + 4, (uint32_t)(r - 1));
}

hipError_t launch_litmus(uint32_t* data, uint32_t* flag, uint32_t* done, uint32_t* res, int rounds, int words,
                         int grid, uint64_t wd_ticks, hipStream_t st) {
  void* args[] = {&data, &flag, &done, &res, &rounds, &words, &wd_ticks};
  return hipLaunchCooperativeKernel((const void*)handoff_litmus, dim3(grid), dim3(NT), args, 0, st);
}

hipError_t litmus_occupancy(int* blocks_per_cu) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, (const void*)handoff_litmus, NT, 0);
}

// ---- the allocation-free variant of the hand-off litmus test -------------------------------
// Its buffers (flag, done and result lines, then the hand-off words) live in `scratch`, a file-scope
// device array of a fixed size that every GPU holds until the process ends. Host code never passes
// the array's name to a kernel (in host code it is a host-side stand-in): the device address of this
// GPU's copy comes from hipGetSymbolAddress, once per device, and only that address is used.
constexpr int LITMUS_CTL_WORDS = 3 * CTR_STRIDE;       // flag, done, result: one 256-byte line each
static __device__ __align__(256) uint32_t scratch[LITMUS_CTL_WORDS + LITMUS_SCRATCH_WORDS];

__global__ void __launch_bounds__(256) fill_zero(uint32_t* p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0u;
}

constexpr int MAX_DEVICES = 64;
static uint32_t* scratch_ptr[MAX_DEVICES];
static std::mutex scratch_mutex;

hipError_t litmus_scratch(uint32_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));   // this device's copy (it is current)
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    scratch_ptr[dev] = static_cast<uint32_t*>(ptr);
  }
  *out = scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_litmus_scratch(uint32_t* base, int rounds, int words, int grid, uint64_t wd_ticks, hipStream_t st) {
  const int n = LITMUS_CTL_WORDS + words;
  hipLaunchKernelGGL(fill_zero, dim3((n + 255) / 256 < 256 ? (n + 255) / 256 : 256), dim3(256), 0, st, base, n);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_litmus(base + LITMUS_CTL_WORDS, base, base + CTR_STRIDE, base + 2 * CTR_STRIDE, rounds, words, grid,
                       wd_ticks, st);
}

int split_max() { return SPLIT_MAX; }
int merge_max() { return MERGE_MAX; }
int out_max_rows() { return OUT_MAXR; }
int down_rows() { return DOWN_ROWS; }

}  // namespace mk
