// Persistent batch-1 fp16 decode monokernel for gfx950 (MI355X).
//
// One launch runs n decode steps of a whole decoder without returning to the
// host: every step does the embedding gather, per layer RMSNorm -> QKV GEMV
// -> RoPE + KV append -> split-context attention -> O GEMV + residual ->
// RMSNorm -> gate/up GEMV + SwiGLU -> down GEMV + residual, then the final
// RMSNorm, the LM-head GEMV and a greedy argmax whose token feeds the next
// step.  This is the "monokernel" of the Kog Inference Engine pages (one
// persistent program for the whole decode loop, no kernel launches between
// layers, grid synchronisations removed, LM-head sampling inside the kernel),
// written for CDNA4:
//
//  * one workgroup per compute unit (grid = CU count, co-resident by
//    cooperative launch), 8 wave64s per workgroup;
//  * every wave streams its slice of the weights (and, for attention, of the
//    KV cache) as 1-KB chunks through a ring of kDepth LDS slots filled by
//    global_load_lds DMAs; the load cursor is wave-uniform (scalar
//    registers) and runs ahead of the consumer across phase boundaries, so
//    weight bytes keep flowing while a wave waits for the activation it
//    needs;
//  * cross-workgroup dependencies use self-validating 64-bit words (32-bit
//    payload + 32-bit step epoch) written and polled with agent-scope relaxed
//    atomics: a consumer waits on the data itself, not on a counter followed
//    by a second read;
//  * the KV cache is written with ordinary stores and ordered once per step by
//    a release fence before each workgroup's end-of-step word and an acquire
//    fence after reading all of them.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "kie_layout.h"

// This file is compiled once per ring depth (KIE_RING_DEPTH, see
// kie_layout.h): each build's code lives in its own namespace and its entry
// points carry the depth in their names.
#define KIE_CAT2(a, b) a##b
#define KIE_CAT(a, b) KIE_CAT2(a, b)
#define KIE_RING_NS KIE_CAT(ring, KIE_RING_DEPTH)
#define KIE_RING_ENTRY(name) KIE_CAT(KIE_CAT(name, _ring), KIE_RING_DEPTH)

namespace kie {
namespace KIE_RING_NS {

typedef unsigned long long u64;
constexpr int kDepth = kRingDepth;  // 1-KB wave units in flight per wave (LDS ring slots)
// s_waitcnt immediate that waits until at most kDepth-1 vector memory
// operations are outstanding (expcnt and lgkmcnt left at their maximum)
constexpr int kWaitRing = ((kDepth - 1) & 15) | (((kDepth - 1) >> 4) << 14) | (7 << 4) | (15 << 8);
constexpr int kWaitRing2 = ((kDepth - 2) & 15) | (((kDepth - 2) >> 4) << 14) | (7 << 4) | (15 << 8);
constexpr int kWaitRing4 = ((kDepth - 4) & 15) | (((kDepth - 4) >> 4) << 14) | (7 << 4) | (15 << 8);
constexpr int kWaitAllVm = (7 << 4) | (15 << 8);
static_assert(kDepth >= 4 && kDepth <= 32, "ring depth");
// s_waitcnt immediate for lgkmcnt(0) only (vmcnt and expcnt at their maximum)
constexpr int kWaitLgkm = 15 | (3 << 14) | (7 << 4);

#define KIE_DI __device__ __forceinline__

// ---------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------
KIE_DI u64 ll_load(const u64* a) { return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
KIE_DI void ll_store(u64* a, uint32_t payload, uint32_t epoch) {
  __hip_atomic_store(a, ((u64)epoch << 32) | (u64)payload, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
KIE_DI void ll_storef(u64* a, float v, uint32_t epoch) { ll_store(a, __float_as_uint(v), epoch); }
KIE_DI uint32_t ll_epoch(u64 w) { return (uint32_t)(w >> 32); }
KIE_DI float ll_f(u64 w) { return __uint_as_float((uint32_t)w); }

template <int CTRL>
KIE_DI float dppf(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// sum over each row of 16 lanes, result in every lane of the row
KIE_DI float row16_sum(float v) {
  v += dppf<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dppf<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dppf<0x141>(v);  // row_half_mirror
  v += dppf<0x140>(v);  // row_mirror
  return v;
}
KIE_DI float readlane_f(float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); }
// full-wave sum, fixed association, uniform result
KIE_DI float wave_sum(float v) {
  v = row16_sum(v);
  return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}
// full-wave maximum (every lane gets it)
KIE_DI float wave_max(float v) {
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}
// sum over groups of `lpk` consecutive lanes; every lane of a group gets it
// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, SC 2011), first output word
// for counter (c0, c1, 0, 0) and key (k0, k1): ten rounds of two 32x32->64
// products, the key advanced by the two Weyl increments after each round
KIE_DI uint32_t philox_w0(uint32_t c0, uint32_t c1, uint32_t k0, uint32_t k1) {
  uint32_t c2 = 0, c3 = 0;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
    const uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
    c0 = hi1 ^ c1 ^ k0;
    c1 = lo1;
    c2 = hi0 ^ c3 ^ k1;
    c3 = lo0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c0;
}
// standard Gumbel noise -log(-log(u)), u = (top 23 bits + 1/2) * 2^-23 in (0, 1)
KIE_DI float gumbel(uint32_t w) {
  const float u = ((float)(w >> 9) + 0.5f) * 0x1p-23f;
  return -logf(-logf(u));
}

// greedy order: the larger value wins, equal values go to the smaller index
KIE_DI bool argmax_better(float ov, int oi, float bv, int bi) { return ov > bv || (ov == bv && oi < bi); }
KIE_DI void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(v, off);
    const int oi = __shfl_xor(i, off);
    if (argmax_better(ov, oi, v, i)) {
      v = ov;
      i = oi;
    }
  }
}
// sum over each key's lpk lanes (dl: this lane's index inside its key)
KIE_DI float group_sum(float v, int lpk, int dl) {
  if (lpk == 16) return row16_sum(v);
  if (lpk == 8) {
    v += dppf<0xB1>(v);
    v += dppf<0x4E>(v);
    v += dppf<0x141>(v);
    return v;
  }
  if (lpk == 4) {
    v += dppf<0xB1>(v);
    v += dppf<0x4E>(v);
    return v;
  }
  if (lpk == 32) {
    v = row16_sum(v);
    return v + __shfl_xor(v, 16);
  }
  // other widths: a tree inside the key (lane dl adds lane dl + o while that
  // is inside the key, o = 1, 2, 4, ...), then the key's first lane holds
  // the sum and broadcasts it
  const int lane = (int)(threadIdx.x & 63);
  for (int o = 1; o < lpk; o *= 2) {
    const float t = __shfl(v, lane + o);
    if (dl + o < lpk) v += t;
  }
  return __shfl(v, lane - dl);
}

KIE_DI float h2f_lo(uint32_t u) { return __half2float(__ushort_as_half((unsigned short)(u & 0xFFFF))); }
KIE_DI float h2f_hi(uint32_t u) { return __half2float(__ushort_as_half((unsigned short)(u >> 16))); }
KIE_DI float hbits2f(uint16_t u) { return __half2float(__ushort_as_half(u)); }

// position of element k of a GEMV input vector in LDS: element 8g + j sits
// in plane j / 4 (planes `plane` floats apart) at float 4g + j % 4, so the
// 16-byte reads of lanes with consecutive g are conflict-free
KIE_DI int xs_pos(int k, int plane) { return ((k >> 2) & 1) * plane + ((k >> 3) << 2) + (k & 3); }

// Wave-uniform values must be provably uniform to the compiler: a value it
// thinks may differ between lanes turns every branch on it into a divergent
// one, and a loop with a possibly divergent exit makes all its loop-carried
// state (the load cursor, the ring slot) per-lane vector values.
KIE_DI int rfl(int v) { return __builtin_amdgcn_readfirstlane(v); }
// A per-lane value the compiler must treat as new at every use: index math
// built on it stays inside the loop that needs it instead of being hoisted to
// the kernel entry, where it would hold registers for the whole launch.
KIE_DI int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// combine (m, l, acc) with (mo, lo, ao); m in log2 units, -inf = empty
KIE_DI void lse_merge(float& m, float& l, float* acc, float mo, float lo, const float* ao) {
  const float mn = fmaxf(m, mo);
  if (mn == -INFINITY) return;
  const float a = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mn);
  const float b = mo == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mo - mn);
  l = a * l + b * lo;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = a * acc[e] + b * ao[e];
  m = mn;
}

// Workgroup barrier for LDS data.  __syncthreads() would also order this
// wave's LDS-DMA ring loads (they write LDS) and so wait for every ring load
// in flight; no other wave reads a wave's ring, so only this wave's ordinary
// LDS accesses must be complete.  The empty asm statements keep the compiler
// from moving memory accesses across the barrier.
KIE_DI void wg_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kWaitLgkm);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// one key into an online softmax: (m, l, acc) += exp2(s - m) * v
KIE_DI void online_update(float& m, float& l, float* acc, float s, const float* v) {
  const float mn = fmaxf(m, s);
  const float scale = (m == mn) ? 1.f : __builtin_amdgcn_exp2f(m - mn);
  const float pv = (s == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s - mn);
  l = l * scale + pv;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = acc[e] * scale + pv * v[e];
  m = mn;
}

// ---------------------------------------------------------------------------
// launch-wide state
// ---------------------------------------------------------------------------
struct Shared {  // small LDS block after the planned area
  int abort;
  int pad[3];
  float redf[kWaves];
  float lmv[kWaves];
  int lmi[kWaves];
  float tokv[kWaves];  // end of step: each wave's best (value, index) over the workgroup partials
  int toki[kWaves];
};
static_assert(sizeof(Shared) <= kSharedReserve, "Shared block");

struct Dev {
  const KParams* p;
  int wg, nwg, wave, lane, tid;
  Shared* sh;
  int* desc;
  uint4* ring;        // this wave's kDepth x 1 KB LDS ring
  uint32_t ring_lane; // LDS byte address of this lane's 16 bytes in ring slot 0
  int lane16;         // lane * 16
  int plane;          // floats between the two planes of a GEMV input
  int32_t* state;
  u64 *X, *Q, *KC, *VC, *REC, *OB, *HB, *LMP;
  const float2* rope;
  uint32_t* tbuf;     // LDS phase stamps of the current step (tracing only)
  int lpk, kpl, kl, dl, lane_active;
};

// The workgroup's abort flag.  It is read and written through an LDS-typed
// pointer: through a generic pointer a volatile access becomes a flat load,
// which also counts as a vector memory access, and its wait then waits for
// every ring load in flight.
typedef __attribute__((address_space(3))) volatile int lds_vint;
KIE_DI lds_vint* abort_flag(const Dev& D) { return (lds_vint*)(__attribute__((address_space(3))) int*)&D.sh->abort; }
KIE_DI bool abort_seen(const Dev& D) { return *abort_flag(D) != 0; }
KIE_DI void set_abort(const Dev& D) { *abort_flag(D) = 1; }
// the abort flag read after a barrier (uniform)
KIE_DI bool aborted(const Dev& D) { return rfl(*abort_flag(D)) != 0; }

KIE_DI void raise_status(const Dev& D, int code) {
  atomicCAS(&D.state[0], 0, code);
  __hip_atomic_store(&D.state[1], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  set_abort(D);
}

// spin on one word until its epoch matches; false on timeout / abort
KIE_DI bool spin_word(const Dev& D, const u64* a, uint32_t epoch, u64* out) {
  const uint64_t t0 = wall_clock64();
  for (int it = 0;; ++it) {
    __builtin_amdgcn_s_sleep(1);
    const u64 w = ll_load(a);
    if (ll_epoch(w) == epoch) {
      *out = w;
      return true;
    }
    if ((it & 15) == 15) {
      if (abort_seen(D)) return false;
      if (__hip_atomic_load(&D.state[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
        set_abort(D);
        return false;
      }
      if (wall_clock64() - t0 > D.p->timeout_ticks) {
        raise_status(D, DEV_TIMEOUT);
        return false;
      }
    }
  }
}

// Race-detection aid (DBG_JITTER): each wave sleeps a pseudo-random time,
// 0 to ~6 us, at the start of every phase, hashed from (workgroup, wave,
// epoch, phase), so every launch reorders the workgroups' arrivals.  Results
// must not change by a single bit: each output has one owner and a fixed
// order of additions.
KIE_DI void jitter(const Dev& D, uint32_t epoch, int ph) {
  uint32_t h = (uint32_t)D.wg * 0x9E3779B1u ^ (uint32_t)D.wave * 0x85EBCA77u ^ epoch * 0xC2B2AE3Du ^
               (uint32_t)ph * 0x27D4EB2Fu;
  h ^= h >> 15;
  h *= 0x2C1B3C6Du;
  h ^= h >> 12;
  const int n = rfl((int)(h & 15));
  for (int i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(16);
}

// Phase trace stamp (thread 0 of the workgroup only).  Stamps go to LDS and
// reach memory at the end of the step: a global store here would be waited
// for by the next vmcnt wait of the wave and move the very times measured.
KIE_DI bool tracing(const Dev& D, int s) { return D.p->trace && s < D.p->trace_steps; }
KIE_DI void stamp(const Dev& D, int s, int ph, int k) {
  if (tracing(D, s) && D.tid == 0) {
    if (!D.tbuf) {  // no room in LDS
      D.p->trace[(((uint64_t)s * kTracePhases + ph) * D.nwg + D.wg) * 4 + k] = wall_clock64();
      return;
    }
    const int L = D.p->m.L;
    const int slot = ph < 5 * 64 ? ph : trace_slots(L) - 1;
    D.tbuf[slot * 4 + k] = (uint32_t)wall_clock64();
  }
}
// (every thread) clear the step's stamps
KIE_DI void trace_begin(const Dev& D, int s) {
  if (!tracing(D, s) || !D.tbuf) return;
  const int n = trace_slots(D.p->m.L) * 4;
  for (int i = D.tid; i < n; i += kThreads) D.tbuf[i] = 0;
}
// (every thread) write the step's stamps to the trace buffer, widened to 64
// bits against the current clock; holds one workgroup barrier
KIE_DI void trace_end(const Dev& D, int s) {
  if (!tracing(D, s) || !D.tbuf) return;
  const int L = D.p->m.L;
  const int n = trace_slots(L) * 4;
  const uint64_t now = wall_clock64();
  for (int i = D.tid; i < n; i += kThreads) {
    const uint32_t lo = D.tbuf[i];
    uint64_t v = 0;
    if (lo) {
      v = (now & ~0xFFFFFFFFull) | lo;
      if (v > now) v -= 1ull << 32;
    }
    const int slot = i >> 2;
    const int ph = slot < trace_slots(L) - 1 ? slot : 5 * 64 + 1;
    D.p->trace[(((uint64_t)s * kTracePhases + ph) * D.nwg + D.wg) * 4 + (i & 3)] = v;
  }
  wg_sync();
}

// Wait until the words base[k*stride] (k < N, mask bit k set) all carry
// `epoch`.  Every round re-issues the loads of all words still stale
// together, so detection costs one memory round trip after the last word
// lands rather than one per word.  Returns false on timeout or abort.
template <int N>
KIE_DI bool poll_words(const Dev& D, const u64* base, int stride, uint32_t mask, uint32_t epoch, u64 (&v)[N]) {
#pragma unroll
  for (int k = 0; k < N; ++k)
    if (mask & (1u << k)) v[k] = ll_load(base + (long)k * stride);
  uint64_t t0 = 0;
  for (int it = 0;; ++it) {
    uint32_t stale = 0;
#pragma unroll
    for (int k = 0; k < N; ++k)
      if ((mask & (1u << k)) && ll_epoch(v[k]) != epoch) stale |= 1u << k;
    if (!stale) return true;
    if (it == 0) t0 = wall_clock64();
    if ((it & 15) == 15) {
      if (abort_seen(D)) return false;
      if (__hip_atomic_load(&D.state[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
        set_abort(D);
        return false;
      }
      if (wall_clock64() - t0 > D.p->timeout_ticks) {
        raise_status(D, DEV_TIMEOUT);
        return false;
      }
    }
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int k = 0; k < N; ++k)
      if (stale & (1u << k)) v[k] = ll_load(base + (long)k * stride);
  }
}

// Wait until the words *a[k] (k < N, mask bit k set) all carry `epoch`, as
// poll_words for scattered addresses.  Returns false on timeout or abort.
template <int N>
KIE_DI bool poll_addrs(const Dev& D, const u64* const (&a)[N], uint32_t mask, uint32_t epoch, u64 (&v)[N]) {
#pragma unroll
  for (int k = 0; k < N; ++k)
    if (mask & (1u << k)) v[k] = ll_load(a[k]);
  uint64_t t0 = 0;
  for (int it = 0;; ++it) {
    uint32_t stale = 0;
#pragma unroll
    for (int k = 0; k < N; ++k)
      if ((mask & (1u << k)) && ll_epoch(v[k]) != epoch) stale |= 1u << k;
    if (!stale) return true;
    if (it == 0) t0 = wall_clock64();
    if ((it & 15) == 15) {
      if (abort_seen(D)) return false;
      if (__hip_atomic_load(&D.state[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
        set_abort(D);
        return false;
      }
      if (wall_clock64() - t0 > D.p->timeout_ticks) {
        raise_status(D, DEV_TIMEOUT);
        return false;
      }
    }
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int k = 0; k < N; ++k)
      if (stale & (1u << k)) v[k] = ll_load(a[k]);
  }
}

// the workgroup polls words [0, n) of src into dst (planes for a GEMV input)
template <bool SWZ>
KIE_DI void poll_to_lds(const Dev& D, const u64* src, float* dst, int n, uint32_t epoch) {
  const int plane = D.plane;
  for (int base = D.tid; base < n; base += kThreads * 8) {
    uint32_t mask = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (base + k * kThreads < n) mask |= 1u << k;
    u64 v[8];
    if (!poll_words<8>(D, src + base, kThreads, mask, epoch, v)) return;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int i = base + k * kThreads;
      if (i < n) dst[SWZ ? xs_pos(i, plane) : i] = ll_f(v[k]);
    }
  }
}

// Up to three vectors polled in one round trip: word j of the concatenation
// (j = tid + k * kThreads, k < K) is loaded for all k before any is waited
// for, and only stale words are loaded again.  Returns false on abort or
// time-out (as poll_words).  The caller checks n0 + n1 + n2 <= K * kThreads.
struct PollSeg {
  const u64* src;
  float* dst;
  int n, swz;
};
template <int K>
KIE_DI bool poll_multi(const Dev& D, const PollSeg (&sg)[3], uint32_t epoch) {
  const int n01 = sg[0].n + sg[1].n, nt = n01 + sg[2].n;
  u64 v[K];
  auto addr = [&](int j) -> const u64* {
    return j < sg[0].n ? sg[0].src + j : j < n01 ? sg[1].src + (j - sg[0].n) : sg[2].src + (j - n01);
  };
  uint32_t mask = 0;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int j = D.tid + k * kThreads;
    if (j < nt) {
      mask |= 1u << k;
      v[k] = ll_load(addr(j));
    }
  }
  uint64_t t0 = 0;
  for (int it = 0;; ++it) {
    uint32_t stale = 0;
#pragma unroll
    for (int k = 0; k < K; ++k)
      if ((mask & (1u << k)) && ll_epoch(v[k]) != epoch) stale |= 1u << k;
    if (!stale) break;
    if (it == 0) t0 = wall_clock64();
    if ((it & 15) == 15) {
      if (abort_seen(D)) return false;
      if (__hip_atomic_load(&D.state[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
        set_abort(D);
        return false;
      }
      if (wall_clock64() - t0 > D.p->timeout_ticks) {
        raise_status(D, DEV_TIMEOUT);
        return false;
      }
    }
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int k = 0; k < K; ++k)
      if (stale & (1u << k)) v[k] = ll_load(addr(D.tid + k * kThreads));
  }
  const int plane = D.plane;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int j = D.tid + k * kThreads;
    if (j < nt) {
      const int s = j < sg[0].n ? 0 : j < n01 ? 1 : 2;
      const int i = j - (s == 0 ? 0 : s == 1 ? sg[0].n : n01);
      sg[s].dst[sg[s].swz ? xs_pos(i, plane) : i] = ll_f(v[k]);
    }
  }
  return true;
}
constexpr int kMultiPoll1 = 14, kMultiPoll2 = 10;  // words per thread of a batched poll (one, two vectors)

// ---------------------------------------------------------------------------
// work descriptors (in LDS, see kie_layout.h)
// ---------------------------------------------------------------------------
KIE_DI int lm_active(const KParams& p, int s) { return p.lm_mode == 0 || (p.lm_mode == 1 && s == p.n_steps - 1); }
KIE_DI int nphases(const KParams& p, int s) { return 5 * p.m.L + (lm_active(p, s) ? 1 : 0); }
KIE_DI int gemv_index(int kind) {
  return kind == PH_QKV ? 0 : kind == PH_O ? 1 : kind == PH_GU ? 2 : kind == PH_DOWN ? 3 : 4;
}
KIE_DI uint64_t matrix_offset(const KParams& p, int kind) {
  return kind == PH_QKV ? p.pl.wqkv : kind == PH_O ? p.pl.wo : kind == PH_GU ? p.pl.wgu : kind == PH_DOWN ? p.pl.wd
                                                                                                             : p.pl.lm_head;
}

// one wave's share of GEMV `kind` -> its 8-int descriptor (and the workgroup's rows)
template <int G>
KIE_DI void write_gemv_desc(const KParams& p, int kind, int nwg, int wg, int wave, int* dsc, int* wgrows) {
  const GemvShape sh = gemv_shape(p.m, kind);
  int r0, r1, c0, c1;
  if constexpr (G > 2) {
    gemv_rows_any(p.m, kind, nwg, wg, &r0, &r1);  // (mergers per query head)
  } else {
    gemv_rows(p.m, kind, nwg, wg, &r0, &r1);
  }
  gemv_wave_chunks(r1 - r0, sh.K, wave, &c0, &c1);
  const int nb = col_blocks(sh.K);
  const uint64_t off = matrix_offset(p, kind) + packed_at((uint64_t)r0, 0, sh.K) + (uint64_t)c0 * kBlock;
  dsc[0] = (int)(uint32_t)off;
  dsc[1] = (int)(uint32_t)(off >> 32);
  dsc[2] = c1 - c0;
  dsc[3] = c0 / nb;  // first row pair (from the workgroup's first row)
  dsc[4] = c0 % nb;  // first column block
  dsc[5] = nb;
  dsc[6] = 0;
  dsc[7] = 0;
  if (wave == 0) {
    wgrows[0] = r0;
    wgrows[1] = r1 - r0;
  }
}

// one wave's attention work at position pos -> 12-int descriptor
template <int G>
KIE_DI void write_attn_desc(const KParams& p, int nwg, int wg, int wave, int kpl, int pos, int* dsc) {
  const int n_ctx = pos + 1;
  AttnSeg seg[2];
  seg[0] = AttnSeg{0, 0, 0};
  seg[1] = AttnSeg{0, 0, 0};
  const int nseg = attn_segments(p.m.Hkv, n_ctx, nwg, wg, seg);
  int merge_g = -1;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    int ka = 0, kc = 0, nst = 0, hp = 0;
    if (s < nseg) {
      int wa, wb;
      wave_split(seg[s].tb - seg[s].ta, wave, &wa, &wb);
      wa += seg[s].ta;
      wb += seg[s].ta;
      ka = wa;
      const int c = wb < pos ? wb : pos;
      kc = c > wa ? c : wa;
      nst = (kc - wa + kpl - 1) / kpl;
      hp = (wa <= pos && pos < wb) ? 1 : 0;
      if (seg[s].tb == n_ctx) merge_g = seg[s].g;
    }
    dsc[5 * s + 0] = seg[s].g;
    dsc[5 * s + 1] = ka;
    dsc[5 * s + 2] = kc;
    dsc[5 * s + 3] = nst;
    dsc[5 * s + 4] = hp;
  }
  if constexpr (G > 2) {
    // one merger per query head (attn_mergers): the group's last G
    // workgroups, workgroup w1 - 1 - h merging head h, coded as
    // g + (h + 1) * 2^16 (a lone merger of every head stays g)
    if (attn_mergers(p.m, nwg) > 1) {
      const int g = attn_head(p.m.Hkv, nwg, wg);
      int w0, w1;
      split(nwg, p.m.Hkv, g, &w0, &w1);
      const int h = w1 - 1 - wg;
      merge_g = h < G ? g + ((h + 1) << 16) : -1;
    }
  }
  dsc[10] = nseg;
  dsc[11] = merge_g;
}

// ---------------------------------------------------------------------------
// the load cursor: walks this wave's chunk sequence (weights and KV rows) and
// issues exactly one 1-KB chunk load into the ring per call.  All of its
// state is wave-uniform, so it lives in scalar registers; a chunk load is a
// scalar address step plus one global_load_lds with the lane's fixed offset.
// ---------------------------------------------------------------------------
struct Cursor {
  uint64_t base;    // byte address of the next chunk (attention: next K chunk)
  uint64_t voff;    // attention: V chunk address minus K chunk address
  uint32_t stride;  // bytes from one chunk (attention: key step) to the next
  int rem;          // chunks left in this stretch (attention: 2 per key step)
  int attn, kvh, seg, ph, nph, done;
  int layer;        // layer of the phase ph
};

// attention segment sg of layer l of this step (an empty one has rem 0)
KIE_DI void cursor_attn_seg(const Dev& D, Cursor& c, int l, int sg) {
  const KParams& p = *D.p;
  const int* a = D.desc + D.wave * kWaveDesc + kConsumerAttn + 5 * sg;
  const int g = rfl(a[0]), ka = rfl(a[1]), nst = rfl(a[3]);
  c.seg = sg;
  c.rem = 2 * nst;
  c.kvh = 0;
  c.base = (uint64_t)(uintptr_t)p.kv + 2 * (kv_offset(p.m, l, 0, g) + (uint64_t)ka * (uint64_t)p.m.hd);
}

KIE_DI void cursor_enter(const Dev& D, Cursor& c) {
  const KParams& p = *D.p;
  int kind = PH_LM, l = 0;
  if (c.ph < 5 * p.m.L) phase_at(p.lp.pipe, p.m.parallel, p.m.L, c.ph, &kind, &l);
  c.layer = l;
  if (kind == PH_ATTN) {
    c.attn = 1;
    c.stride = (uint32_t)(attn_kpl(p.m.hd) * p.m.hd * 2);
    c.voff = 2 * (kv_offset(p.m, 0, 1, 0) - kv_offset(p.m, 0, 0, 0));
    cursor_attn_seg(D, c, l, 0);
    return;
  }
  const int* g = D.desc + D.wave * kWaveDesc + 8 * gemv_index(kind);
  const uint64_t off = (uint64_t)(uint32_t)rfl(g[0]) | ((uint64_t)(uint32_t)rfl(g[1]) << 32);
  c.attn = 0;
  c.kvh = 0;
  c.seg = 0;
  c.voff = 0;
  c.stride = kChunkBytes;
  c.base = (uint64_t)(uintptr_t)p.W + 2 * ((kind == PH_LM ? 0 : (uint64_t)l * p.pl.layer_stride) + off);
  c.rem = rfl(g[2]);
}

// The cursor never crosses into the next step by itself: the next step reads
// KV-cache rows written during this step, which are only visible after the
// end-of-step acquire.  At the end of its step it issues harmless loads until
// the consumer restarts it after that acquire.
KIE_DI void cursor_advance(const Dev& D, Cursor& c) {
  while (c.rem == 0 && !c.done) {
    if (c.attn && c.seg == 0) {
      cursor_attn_seg(D, c, c.layer, 1);
      continue;
    }
    if (++c.ph >= c.nph) {
      c.done = 1;
      break;
    }
    cursor_enter(D, c);
  }
}

KIE_DI void dma_chunk(const Dev& D, uint64_t a, int slot);

// issue the next chunk into ring slot `slot` (one DMA per call).  A chunk
// may run past the end of its stretch (the last one of a workgroup's rows,
// keys past the context, lanes past the keys of a step); those bytes stay in
// the buffer (it ends in a zero tail) and the consumer discards them.
KIE_DI void cursor_issue(const Dev& D, Cursor& c, int slot) {
  if (c.rem == 0) cursor_advance(D, c);
  uint64_t a = (uint64_t)(uintptr_t)D.p->W;  // after the step: the first packed kilobyte
  if (!c.done) {
    a = c.base + (c.kvh ? c.voff : 0);
    if (c.kvh || !c.attn) c.base += c.stride;
    c.kvh ^= c.attn;
    --c.rem;
  }
  dma_chunk(D, a, slot);
}

// Re-assert that the cursor and the ring slot are wave-uniform (they are;
// readfirstlane makes it visible to the compiler, so the stream loops keep
// them in scalar registers and branch on them with scalar branches).
KIE_DI uint64_t rfl64(uint64_t v) {
  return (uint64_t)(uint32_t)rfl((int)(uint32_t)v) | ((uint64_t)(uint32_t)rfl((int)(uint32_t)(v >> 32)) << 32);
}
KIE_DI void make_uniform(Cursor& c, int& slot) {
  c.base = rfl64(c.base);
  c.voff = rfl64(c.voff);
  c.stride = (uint32_t)rfl((int)c.stride);
  c.rem = rfl(c.rem);
  c.attn = rfl(c.attn);
  c.kvh = rfl(c.kvh);
  c.seg = rfl(c.seg);
  c.ph = rfl(c.ph);
  c.nph = rfl(c.nph);
  c.done = rfl(c.done);
  slot = rfl(slot);
}

KIE_DI int ring_next(int s) { return s + 1 == kDepth ? 0 : s + 1; }
KIE_DI int ring_add(int s, int k) { return s + k >= kDepth ? s + k - kDepth : s + k; }
KIE_DI uint32_t ring_addr(const Dev& D, int slot) { return D.ring_lane + (uint32_t)slot * kChunkBytes; }

KIE_DI void dma_chunk(const Dev& D, uint64_t a, int slot) {
  // 16 bytes per lane straight into LDS: lane i lands at slot + 16 i
  __builtin_amdgcn_global_load_lds((const void*)((const char*)(uintptr_t)a + D.lane16),
                                   (__attribute__((address_space(3))) void*)(D.ring + slot * kWave), 16, 0,
                                   2 /* nt */);
}

// issue the next four chunks into slots slot .. slot+3.  Inside one stretch
// (four GEMV chunks, or two whole attention key steps) that is four scalar
// address steps; otherwise it falls back to one cursor_issue per chunk.
KIE_DI void cursor_issue4(const Dev& D, Cursor& c, int slot) {
  if (!c.done && c.rem >= 4 && c.kvh == 0) {
    const uint64_t b = c.base;
    const uint64_t s1 = c.attn ? c.voff : (uint64_t)kChunkBytes;
    const uint64_t s2 = c.attn ? (uint64_t)c.stride : 2ull * kChunkBytes;
    dma_chunk(D, b, slot);
    dma_chunk(D, b + s1, ring_add(slot, 1));
    dma_chunk(D, b + s2, ring_add(slot, 2));
    dma_chunk(D, b + s2 + s1, ring_add(slot, 3));
    c.base = b + 2 * s2;
    c.rem -= 4;
  } else {
#pragma unroll 1
    for (int k = 0; k < 4; ++k) cursor_issue(D, c, ring_add(slot, k));
  }
}

// Refills owed by the attention stream.  Once the cursor has left the
// attention chunks, the attention stream stops refilling the slots it frees:
// those loads (the next phase's first weights) would queue in front of the
// merger's record poll and the next prologue's poll (a wave's loads complete
// in issue order), and issuing them while the memory pipeline is full would
// stall the attention arithmetic itself.  They are issued after the
// attention records are out, into the consecutive slots from `slot`.
struct Owed {
  int n, slot;
};
// refill the k freed slots from `slot` on: attention chunks while the
// cursor still has some (it is not advanced here), the rest owed
KIE_DI void attn_refill(const Dev& D, Cursor& c, int slot, int k, Owed& o) {
  int i = 0;
  if (o.n == 0 && c.attn && !c.done) {
#pragma unroll 1
    for (; i < k && c.rem > 0; ++i) {
      dma_chunk(D, c.base + (c.kvh ? c.voff : 0), ring_add(slot, i));
      if (c.kvh) c.base += c.stride;
      c.kvh ^= 1;
      --c.rem;
    }
  }
  if (i < k) {
    if (o.n == 0) o.slot = ring_add(slot, i);
    o.n += k - i;
  }
}
KIE_DI void issue_owed(const Dev& D, Cursor& c, Owed& o) {
  make_uniform(c, o.slot);
  o.n = rfl(o.n);
#pragma unroll 1
  for (int i = 0; i < o.n; ++i) cursor_issue(D, c, ring_add(o.slot, i));
  o.n = 0;
}

typedef float f4v __attribute__((ext_vector_type(4)));
typedef unsigned u4v __attribute__((ext_vector_type(4)));

// LDS reads of ring slots are written as asm that waits for itself: the
// compiler then neither sees an LDS access that an in-flight ring DMA could
// alias (it would drain every DMA first) nor leaves an output register in
// flight.  A GEMV chunk reads its weights and the lane's two input halves in
// one round trip.
KIE_DI void read_w_x(uint32_t ra, uint32_t xa, uint32_t xb, u4v& w, f4v& a, f4v& b) {
  asm volatile(
      "ds_read_b128 %0, %3\n\t"
      "ds_read_b128 %1, %4\n\t"
      "ds_read_b128 %2, %5\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(w), "=&v"(a), "=&v"(b)
      : "v"(ra), "v"(xa), "v"(xb)
      : "memory");
}
// four GEMV chunks: weights of four ring slots and the input halves of each
KIE_DI void read_w_x4(const uint32_t (&r)[4], const uint32_t (&x)[8], u4v (&w)[4], f4v (&a)[4], f4v (&b)[4]) {
  asm volatile(
      "ds_read_b128 %0, %12\n\t"
      "ds_read_b128 %4, %16\n\t"
      "ds_read_b128 %8, %17\n\t"
      "ds_read_b128 %1, %13\n\t"
      "ds_read_b128 %5, %18\n\t"
      "ds_read_b128 %9, %19\n\t"
      "ds_read_b128 %2, %14\n\t"
      "ds_read_b128 %6, %20\n\t"
      "ds_read_b128 %10, %21\n\t"
      "ds_read_b128 %3, %15\n\t"
      "ds_read_b128 %7, %22\n\t"
      "ds_read_b128 %11, %23\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3]), "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]),
        "=&v"(b[0]), "=&v"(b[1]), "=&v"(b[2]), "=&v"(b[3])
      : "v"(r[0]), "v"(r[1]), "v"(r[2]), "v"(r[3]), "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]),
        "v"(x[6]), "v"(x[7])
      : "memory");
}
// two attention key steps: K, V, K, V of four consecutive slots
KIE_DI void read_kv2(const uint32_t (&r)[4], u4v (&x)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3])
      : "v"(r[0]), "v"(r[1]), "v"(r[2]), "v"(r[3])
      : "memory");
}
KIE_DI void read_kv(uint32_t rk, uint32_t rv, u4v& k, u4v& v) {
  asm volatile(
      "ds_read_b128 %0, %2\n\t"
      "ds_read_b128 %1, %3\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k), "=&v"(v)
      : "v"(rk), "v"(rv)
      : "memory");
}

KIE_DI void unpack8(const u4v x, float* v) {
  v[0] = h2f_lo(x.x); v[1] = h2f_hi(x.x); v[2] = h2f_lo(x.y); v[3] = h2f_hi(x.y);
  v[4] = h2f_lo(x.z); v[5] = h2f_hi(x.z); v[6] = h2f_lo(x.w); v[7] = h2f_hi(x.w);
}

// ---------------------------------------------------------------------------
// GEMV stream: consume this wave's nch chunks of the workgroup's row pairs
// (the first is column block b of pair P; nb blocks per pair) and write one
// partial sum per (row, wave) into part.  Lanes 0..31 accumulate row 2P and
// lanes 32..63 row 2P+1 over the pair's blocks; the cross-lane sums happen
// when the pair (or the wave's share of it) ends.
// ---------------------------------------------------------------------------
// one chunk's 8 products for this lane, summed as two independent chains
KIE_DI float dot_chunk(const u4v w, const f4v a, const f4v b) {
  float t0 = h2f_lo(w.x) * a.x;
  float t1 = h2f_lo(w.z) * b.x;
  t0 = __builtin_fmaf(h2f_hi(w.x), a.y, t0);
  t1 = __builtin_fmaf(h2f_hi(w.z), b.y, t1);
  t0 = __builtin_fmaf(h2f_lo(w.y), a.z, t0);
  t1 = __builtin_fmaf(h2f_lo(w.w), b.z, t1);
  t0 = __builtin_fmaf(h2f_hi(w.y), a.w, t0);
  t1 = __builtin_fmaf(h2f_hi(w.w), b.w, t1);
  return t0 + t1;
}

struct GemvAcc {
  float* part;
  float A;  // this lane's sum for its row of pair P over the blocks so far
  int P, b, nb, wave, lane;
  // the pair's two row sums: a 16-lane sum in every row of the wave, then
  // row 1 adds row 0 and row 3 adds row 2 (row_bcast:15); lane 31 holds row
  // 2P, lane 63 row 2P+1
  KIE_DI void flush() {
    const float r = row16_sum(A);
    const float s = r + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(r), 0x142, 0xA, 0xF, false));
    if ((lane & 31) == 31) part[(2 * P + (lane >> 5)) * kWaves + wave] = s;
    A = 0.f;
    b = 0;
    ++P;
  }
  KIE_DI void fold(float t) {
    A += t;
    if (++b == nb) flush();
  }
};

KIE_DI void gemv_stream(const Dev& D, Cursor& cur, int& slot, const float* xs, float* part, int nch, int P, int b,
                        int nb) {
  make_uniform(cur, slot);
  // this lane's input columns 8 * (lane % 32) .. +8 of block 0: a float4 in
  // each plane (lanes l and l + 32 read the same words)
  const uint32_t xl = (uint32_t)(uintptr_t)xs + (uint32_t)(D.lane & 31) * 16u;
  const uint32_t pb = (uint32_t)D.plane * 4u;
  GemvAcc g{part, 0.f, P, b, nb, D.wave, D.lane};
  int j = 0;
  // four chunks per LDS round trip
  for (; j + 4 <= nch; j += 4) {
    uint32_t ra[4], xa[8];
    int bb = g.b;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      xa[2 * k] = xl + (uint32_t)bb * 512u;
      xa[2 * k + 1] = xa[2 * k] + pb;
      bb = bb + 1 == nb ? 0 : bb + 1;
      ra[k] = ring_addr(D, ring_add(slot, k));
    }
    __builtin_amdgcn_s_waitcnt(kWaitRing4);
    u4v w[4];
    f4v a[4], c[4];
    read_w_x4(ra, xa, w, a, c);
    cursor_issue4(D, cur, slot);
    slot = ring_add(slot, 4);
    float t[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) t[k] = dot_chunk(w[k], a[k], c[k]);
#pragma unroll
    for (int k = 0; k < 4; ++k) g.fold(t[k]);
  }
  for (; j < nch; ++j) {
    const uint32_t xa = xl + (uint32_t)g.b * 512u;
    __builtin_amdgcn_s_waitcnt(kWaitRing);
    u4v w;
    f4v a, c;
    read_w_x(ring_addr(D, slot), xa, xa + pb, w, a, c);
    cursor_issue(D, cur, slot);
    slot = ring_next(slot);
    g.fold(dot_chunk(w, a, c));
  }
  if (g.b > 0) g.flush();
}

// ---------------------------------------------------------------------------
// attention stream: nst key steps of one segment; a step is a K chunk and a
// V chunk of the same kpl keys (lpk lanes per key, 8 dims per lane), folded
// into every key slot's online softmax
// ---------------------------------------------------------------------------
template <int G>
KIE_DI void attn_step(const Dev& D, const u4v kx, const u4v vx, int key, int kc, const float (&q)[G][8],
                      float (&mrow)[G], float (&lrow)[G], float (&acc)[G][8]) {
  const bool ok = D.lane_active && key < kc;
  float k8[8], v8[8];
  unpack8(kx, k8);
  unpack8(vx, v8);
#pragma unroll
  for (int e = 0; e < 8; ++e) v8[e] = ok ? v8[e] : 0.f;  // bytes past the keys may be anything
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float t = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) t = __builtin_fmaf(k8[e], q[h][e], t);
    t = group_sum(t, D.lpk, D.dl);
    online_update(mrow[h], lrow[h], acc[h], ok ? t : -INFINITY, v8);
  }
}

// Two key steps whose keys all lie below kc (wave-uniform: the caller
// checks), folded into each query head's online softmax with one rescale:
// m' = max(m, s0, s1), acc' = acc 2^(m - m') + p0 v0 + p1 v1 with
// p = 2^(s - m').  Every score is finite, so 2^(m - m') needs no guard
// (it is 0 while m is still -inf, and 1 when the maximum stays), and the V
// halves feed the FMAs directly.
template <int G>
KIE_DI void attn_step2_full(const Dev& D, const u4v k0, const u4v v0, const u4v k1, const u4v v1,
                            const float (&q)[G][8], float (&mrow)[G], float (&lrow)[G], float (&acc)[G][8]) {
  const uint32_t vw0[4] = {v0.x, v0.y, v0.z, v0.w}, vw1[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float t0 = dot_chunk(k0, f4v{q[h][0], q[h][1], q[h][2], q[h][3]}, f4v{q[h][4], q[h][5], q[h][6], q[h][7]});
    float t1 = dot_chunk(k1, f4v{q[h][0], q[h][1], q[h][2], q[h][3]}, f4v{q[h][4], q[h][5], q[h][6], q[h][7]});
    t0 = group_sum(t0, D.lpk, D.dl);
    t1 = group_sum(t1, D.lpk, D.dl);
    const float mn = fmaxf(mrow[h], fmaxf(t0, t1));
    const float sc = __builtin_amdgcn_exp2f(mrow[h] - mn);
    const float p0 = __builtin_amdgcn_exp2f(t0 - mn);
    const float p1 = __builtin_amdgcn_exp2f(t1 - mn);
    lrow[h] = __builtin_fmaf(lrow[h], sc, p0 + p1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[h][2 * j] = __builtin_fmaf(p1, h2f_lo(vw1[j]), __builtin_fmaf(p0, h2f_lo(vw0[j]), acc[h][2 * j] * sc));
      acc[h][2 * j + 1] =
          __builtin_fmaf(p1, h2f_hi(vw1[j]), __builtin_fmaf(p0, h2f_hi(vw0[j]), acc[h][2 * j + 1] * sc));
    }
    mrow[h] = mn;
  }
}

// attn_step2_full with the key's lane count LPK fixed at compile time
// (0: the run-time width), for the heads-per-KV-head counts whose key loop
// is bound by vector instructions
template <int LPK>
KIE_DI float group_sum_t(const Dev& D, float v) {
  if constexpr (LPK == 16) {
    return row16_sum(v);
  } else {
    return group_sum(v, D.lpk, D.dl);
  }
}
template <int G, int LPK>
KIE_DI void attn_step2_full_t(const Dev& D, const u4v k0, const u4v v0, const u4v k1, const u4v v1,
                              const float (&q)[G][8], float (&mrow)[G], float (&lrow)[G], float (&acc)[G][8]) {
  const uint32_t vw0[4] = {v0.x, v0.y, v0.z, v0.w}, vw1[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float t0 = dot_chunk(k0, f4v{q[h][0], q[h][1], q[h][2], q[h][3]}, f4v{q[h][4], q[h][5], q[h][6], q[h][7]});
    float t1 = dot_chunk(k1, f4v{q[h][0], q[h][1], q[h][2], q[h][3]}, f4v{q[h][4], q[h][5], q[h][6], q[h][7]});
    t0 = group_sum_t<LPK>(D, t0);
    t1 = group_sum_t<LPK>(D, t1);
    const float mn = fmaxf(mrow[h], fmaxf(t0, t1));
    const float sc = __builtin_amdgcn_exp2f(mrow[h] - mn);
    const float p0 = __builtin_amdgcn_exp2f(t0 - mn);
    const float p1 = __builtin_amdgcn_exp2f(t1 - mn);
    lrow[h] = __builtin_fmaf(lrow[h], sc, p0 + p1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[h][2 * j] = __builtin_fmaf(p1, h2f_lo(vw1[j]), __builtin_fmaf(p0, h2f_lo(vw0[j]), acc[h][2 * j] * sc));
      acc[h][2 * j + 1] =
          __builtin_fmaf(p1, h2f_hi(vw1[j]), __builtin_fmaf(p0, h2f_hi(vw0[j]), acc[h][2 * j + 1] * sc));
    }
    mrow[h] = mn;
  }
}
// the whole pairs of key steps [st, nfull) of a segment, all inside the
// context, through attn_step2_full_t (see attn_stream)
template <int G, int LPK>
KIE_DI void attn_pairs_full(const Dev& D, Cursor& cur, int& slot, Owed& owed, int& st, int nfull,
                            const float (&q)[G][8], float (&mrow)[G], float (&lrow)[G], float (&acc)[G][8]) {
  for (; st < nfull; st += 2) {
    uint32_t ra[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) ra[k] = ring_addr(D, ring_add(slot, k));
    if (rfl(owed.n) == 0) {
      __builtin_amdgcn_s_waitcnt(kWaitRing4);
    } else {
      __builtin_amdgcn_s_waitcnt(kWaitAllVm);
    }
    u4v x[4];
    read_kv2(ra, x);
    if (owed.n == 0 && cur.attn && !cur.done && cur.rem >= 4 && cur.kvh == 0) {
      cursor_issue4(D, cur, slot);
    } else {
      attn_refill(D, cur, slot, 4, owed);
    }
    slot = ring_add(slot, 4);
    attn_step2_full_t<G, LPK>(D, x[0], x[1], x[2], x[3], q, mrow, lrow, acc);
  }
}

// A merger's poll of its group's records into LDS (record r, head h at
// recs[(r * G + h) * (hd + 2) ...]) with K words per thread per round
// trip, for more than two query heads per KV head: those records hold G
// heads each, and in batches of eight words a 32-record group takes five
// round trips one after the other.  Word offsets are kept as 32 bits from
// the record buffer.  A missing record reads as empty (m = -inf); on abort
// or time-out the loop stops (the caller checks after its barrier).
template <int K>
KIE_DI void merger_poll_wide(const Dev& D, int l, int w_first, int nrec, int rw, int wpr, int hoff, int hd,
                             const float* mlw, float* recs, uint32_t epoch) {
  // words [hoff, hoff + wpr) of each record (of rw words) go to recs[r * wpr ...]
  const int n = nrec * wpr;
  for (int base = D.tid; base < n; base += kThreads * K) {
    uint32_t off[K];
    uint32_t mask = 0;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int i = base + k * kThreads;
      off[k] = 0;
      if (i < n) {
        const int r = i / wpr, o = i % wpr;
        const int si = (int)mlw[r * 8 + 7];
        if (si >= 0) {
          off[k] = (uint32_t)((((uint64_t)l * D.nwg + w_first + r) * 2 + si) * rw + hoff + o);
          mask |= 1u << k;
        }
      }
    }
    u64 vv[K];
#pragma unroll
    for (int k = 0; k < K; ++k)
      if (mask & (1u << k)) vv[k] = ll_load(D.REC + off[k]);
    const uint64_t t0 = wall_clock64();
    for (int it = 0;; ++it) {
      uint32_t stale = 0;
#pragma unroll
      for (int k = 0; k < K; ++k)
        if ((mask & (1u << k)) && ll_epoch(vv[k]) != epoch) stale |= 1u << k;
      if (!stale) break;
      if ((it & 15) == 15) {
        if (abort_seen(D)) break;
        if (__hip_atomic_load(&D.state[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
          set_abort(D);
          break;
        }
        if (wall_clock64() - t0 > D.p->timeout_ticks) {
          raise_status(D, DEV_TIMEOUT);
          break;
        }
      }
      __builtin_amdgcn_s_sleep(1);
#pragma unroll
      for (int k = 0; k < K; ++k)
        if (stale & (1u << k)) vv[k] = ll_load(D.REC + off[k]);
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int i = base + k * kThreads;
      if (i < n) {
        float v = 0.f;
        if (mask & (1u << k)) {
          v = ll_f(vv[k]);
        } else if ((i % wpr) % (hd + 2) == 0) {
          v = -INFINITY;  // missing record: empty
        }
        recs[i] = v;
      }
    }
  }
}

template <int G>
KIE_DI void attn_stream(const Dev& D, Cursor& cur, int& slot, Owed& owed, int nst, int ka, int kc,
                        const float (&q)[G][8], float (&mrow)[G], float (&lrow)[G], float (&acc)[G][8]) {
  make_uniform(cur, slot);
  int st = 0;
  if constexpr (G > 2) {
    // More than two query heads per KV head: the pairs of key steps that lie
    // wholly inside the context go first, through the fused two-key update,
    // then the rest (the loop below).  One loop body holding both forms
    // needs more registers than the kernel has; per key, the separate
    // update costs about twice the vector instructions, which made the
    // attention of four query heads per KV head arithmetic-bound.  The
    // key's lane count is fixed per loop (16 lanes for head_dim 128), so
    // the per-key sums carry no width dispatch.
    const int nk = (kc - ka) / D.kpl;  // key steps wholly inside the context
    const int nfull = rfl(imax(0, nk < nst ? nk : nst) & ~1);
    if (D.lpk == 16) {
      attn_pairs_full<G, 16>(D, cur, slot, owed, st, nfull, q, mrow, lrow, acc);
    } else {
      attn_pairs_full<G, 0>(D, cur, slot, owed, st, nfull, q, mrow, lrow, acc);
    }
  }
  for (; st + 2 <= nst; st += 2) {
    uint32_t ra[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) ra[k] = ring_addr(D, ring_add(slot, k));
    // with refills owed fewer loads are in flight than the ring holds, so
    // the usual count no longer marks these slots: wait for all of them
    if (rfl(owed.n) == 0) {
      __builtin_amdgcn_s_waitcnt(kWaitRing4);
    } else {
      __builtin_amdgcn_s_waitcnt(kWaitAllVm);
    }
    u4v x[4];
    read_kv2(ra, x);
    if (owed.n == 0 && cur.attn && !cur.done && cur.rem >= 4 && cur.kvh == 0) {
      cursor_issue4(D, cur, slot);
    } else {
      attn_refill(D, cur, slot, 4, owed);
    }
    slot = ring_add(slot, 4);
    // (four query heads per KV head would run out of registers with both
    // forms inlined)
    if (G <= 2 && ka + (st + 2) * D.kpl <= kc) {
      attn_step2_full<G>(D, x[0], x[1], x[2], x[3], q, mrow, lrow, acc);
    } else {
      attn_step<G>(D, x[0], x[1], ka + st * D.kpl + D.kl, kc, q, mrow, lrow, acc);
      attn_step<G>(D, x[2], x[3], ka + (st + 1) * D.kpl + D.kl, kc, q, mrow, lrow, acc);
    }
  }
  if (st < nst) {
    if (rfl(owed.n) == 0) {
      __builtin_amdgcn_s_waitcnt(kWaitRing2);
    } else {
      __builtin_amdgcn_s_waitcnt(kWaitAllVm);
    }
    const int sv = ring_next(slot);
    u4v kx, vx;
    read_kv(ring_addr(D, slot), ring_addr(D, sv), kx, vx);
    attn_refill(D, cur, slot, 2, owed);
    slot = ring_next(sv);
    attn_step<G>(D, kx, vx, ka + st * D.kpl + D.kl, kc, q, mrow, lrow, acc);
  }
}

// ---------------------------------------------------------------------------
// prologue helpers
// ---------------------------------------------------------------------------
// this thread's RMSNorm gains (elements tid + k * kThreads), loaded into
// registers before the input is polled so that their latency overlaps it.
// The loads are unconditional (a clamped index) and the raw half bits stay
// unconverted until use: a load whose value is used inside its own branch
// gets a wait for it right there, and the loads would run one at a time.
KIE_DI void load_gains(const Dev& D, const uint16_t* g, uint16_t (&gr)[kGainRegs]) {
  const int d = D.p->m.d;
  const int t = opaque(D.tid);
#pragma unroll
  for (int k = 0; k < kGainRegs; ++k) {
    const int i = t + k * kThreads;
    gr[k] = g[i < d ? i : 0];
  }
  asm volatile("" ::: "memory");  // issue the loads here, ahead of the poll
}

// n halves from global memory into LDS as whole 1-KB chunks by LDS DMA,
// the chunks spread over the waves (a chunk may read past the vector: the
// packed buffer continues, and the extra halves are never used)
KIE_DI int gains_pad(int d) { return (d + kBlock - 1) / kBlock * kBlock; }
KIE_DI void copy_halves(const Dev& D, const uint16_t* g, uint16_t* dst, int n) {
  const int nch = (n + kBlock - 1) / kBlock;
#pragma unroll 1
  for (int c = D.wave; c < nch; c += kWaves)
    __builtin_amdgcn_global_load_lds((const void*)((const char*)(g + (uint64_t)c * kBlock) + D.lane16),
                                     (__attribute__((address_space(3))) void*)(dst + c * kBlock), 16, 0, 0);
}
// gains kept in LDS (element i at g[i]), read the way load_gains reads them
KIE_DI void stashed_gains(const Dev& D, const uint16_t* g, uint16_t (&gr)[kGainRegs]) {
  const int d = D.p->m.d;
#pragma unroll
  for (int k = 0; k < kGainRegs; ++k) {
    const int i = D.tid + k * kThreads;
    gr[k] = g[i < d ? i : 0];
  }
}

// xraw -> xs = g * x / sqrt(mean(x^2) + eps) in the two-plane layout, zero
// up to the padded row length
// This thread's elements are read from LDS once, all together (a loop that
// re-read xraw between writes to xs would wait out one LDS round trip per
// element: the compiler cannot tell the two arrays apart).
KIE_DI void rmsnorm_to_xs(const Dev& D, const float* xraw, const uint16_t (&gr)[kGainRegs], float* xs) {
  const KParams& p = *D.p;
  const int d = p.m.d;
  const int t = opaque(D.tid);
  float xv[kGainRegs];
#pragma unroll
  for (int k = 0; k < kGainRegs; ++k) {
    const int i = t + k * kThreads;
    xv[k] = xraw[i < d ? i : 0];
  }
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < kGainRegs; ++k) ss += t + k * kThreads < d ? xv[k] * xv[k] : 0.f;
  ss = wave_sum(ss);
  if (D.lane == 0) D.sh->redf[D.wave] = ss;
  wg_sync();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) tot += D.sh->redf[w];
  const float inv = 1.0f / sqrtf(tot / (float)d + p.m.eps);
  const int padded = padded_cols(d);
#pragma unroll
  for (int k = 0; k < kGainRegs; ++k) {
    const int i = t + k * kThreads;
    if (i < padded) xs[xs_pos(i, D.plane)] = i < d ? xv[k] * inv * hbits2f(gr[k]) : 0.f;
  }
}

// RMSNorm with the scale left to the epilogue:
// W (g * x / rms) = (W (g * x)) / rms, so the prologue writes g * x and each
// wave's sum of squares (to redf), and the epilogue, after the barrier it
// has anyway, multiplies the outputs by rms_inv.  No barrier or second pass
// sits between the input and the stream.
KIE_DI void gain_to_xs(const Dev& D, const float* xraw, const uint16_t (&gr)[kGainRegs], float* xs) {
  const int d = D.p->m.d;
  const int t = opaque(D.tid);
  float xv[kGainRegs];
#pragma unroll
  for (int k = 0; k < kGainRegs; ++k) {
    const int i = t + k * kThreads;
    xv[k] = xraw[i < d ? i : 0];
  }
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < kGainRegs; ++k) ss += t + k * kThreads < d ? xv[k] * xv[k] : 0.f;
  ss = wave_sum(ss);
  if (D.lane == 0) D.sh->redf[D.wave] = ss;
  const int padded = padded_cols(d);
#pragma unroll
  for (int k = 0; k < kGainRegs; ++k) {
    const int i = t + k * kThreads;
    if (i < padded) xs[xs_pos(i, D.plane)] = i < d ? xv[k] * hbits2f(gr[k]) : 0.f;
  }
}
// 1 / sqrt(mean(x^2) + eps) from the waves' sums (after a barrier)
KIE_DI float rms_inv(const Dev& D) {
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) tot += D.sh->redf[w];
  return 1.0f / sqrtf(tot / (float)D.p->m.d + D.p->m.eps);
}

// the same for two gain vectors at once (the parallel block's QKV and
// gate/up read the same x_l): xa = ga * x, xb = gb * x, scale deferred
KIE_DI void gain2_to_xs(const Dev& D, const float* xraw, const uint16_t (&ga)[kGainRegs], float* xa,
                        const uint16_t (&gb)[kGainRegs], float* xb) {
  const int d = D.p->m.d;
  const int t = opaque(D.tid);
  float xv[kGainRegs];
#pragma unroll
  for (int k = 0; k < kGainRegs; ++k) {
    const int i = t + k * kThreads;
    xv[k] = xraw[i < d ? i : 0];
  }
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < kGainRegs; ++k) ss += t + k * kThreads < d ? xv[k] * xv[k] : 0.f;
  ss = wave_sum(ss);
  if (D.lane == 0) D.sh->redf[D.wave] = ss;
  const int padded = padded_cols(d);
#pragma unroll
  for (int k = 0; k < kGainRegs; ++k) {
    const int i = t + k * kThreads;
    if (i < padded) {
      xa[xs_pos(i, D.plane)] = i < d ? xv[k] * hbits2f(ga[k]) : 0.f;
      xb[xs_pos(i, D.plane)] = i < d ? xv[k] * hbits2f(gb[k]) : 0.f;
    }
  }
}


// the zero columns of a padded row (padded_cols(K) > K)
KIE_DI void zero_tail(const Dev& D, float* xs, int K) {
  const int padded = padded_cols(K);
  for (int i = K + D.tid; i < padded; i += kThreads) xs[xs_pos(i, D.plane)] = 0.f;
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
template <int G, bool PAR>
__global__ void __launch_bounds__(kThreads, 1) kie_monokernel(const KParams P) {
  // Two separate LDS objects: the ring, written only by DMAs and read only by
  // the ring-read asm, and everything else.  Keeping them apart lets the compiler
  // prove that ordinary LDS accesses never alias an in-flight ring DMA.
  __shared__ float lds_main[kMainFloats];
  __shared__ Shared sh_static;
  __shared__ uint4 ring_lds[kWaves * kDepth * kWave];
  float* const lds_dyn = lds_main;
  const KParams& p = P;
  Dev D;
  D.p = &P;
  D.tid = threadIdx.x;
  D.nwg = gridDim.x;
  // The work partition numbers the workgroups XCD by XCD: the dispatcher
  // places workgroup b on XCD b % 8, so index (b % 8) * (nwg / 8) + b / 8
  // makes every contiguous range of the partition (a KV head's attention
  // group and its merger, a stretch of GEMV rows) sit on one XCD.
  D.wg = (D.nwg % 8 == 0) ? (int)(blockIdx.x % 8) * (D.nwg / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
  D.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  D.lane = threadIdx.x & 63;
  D.sh = &sh_static;
  D.ring = ring_lds + D.wave * kDepth * kWave;
  D.ring_lane = (uint32_t)(uintptr_t)(D.ring + D.lane);
  D.lane16 = D.lane * 16;
  D.plane = p.lp.kmax / 2;
  D.desc = (int*)(lds_dyn + p.lp.desc);
  D.state = (int32_t*)(p.ws + p.wl.state);
  D.X = (u64*)(p.ws + p.wl.X);
  D.Q = (u64*)(p.ws + p.wl.Q);
  D.KC = (u64*)(p.ws + p.wl.KC);
  D.VC = (u64*)(p.ws + p.wl.VC);
  D.REC = (u64*)(p.ws + p.wl.REC);
  D.OB = (u64*)(p.ws + p.wl.OB);
  D.HB = (u64*)(p.ws + p.wl.HB);
  D.LMP = (u64*)(p.ws + p.wl.LMP);
  D.rope = (const float2*)(p.ws + p.wl.rope);
  D.tbuf = p.lp.trace >= 0 ? (uint32_t*)(lds_dyn + p.lp.trace) : nullptr;
  D.lpk = attn_lpk(p.m.hd);
  D.kpl = attn_kpl(p.m.hd);
  D.kl = D.lane / D.lpk;
  D.dl = D.lane % D.lpk;
  D.lane_active = D.lane < D.kpl * D.lpk;

  const int L = p.m.L, d = p.m.d, H = p.m.H, Hkv = p.m.Hkv, hd = p.m.hd, F = p.m.F, V = p.m.V;
  const int qd = H * hd, kvd = Hkv * hd;
  float* xraw = lds_dyn + p.lp.xraw;
  float* xs = lds_dyn + p.lp.gemv_xs;
  float* part = lds_dyn + p.lp.gemv_part;
  float* wrec = lds_dyn + p.lp.attn_wrec;
  float* mlw = lds_dyn + p.lp.attn_ml;
  float* own = lds_dyn + p.lp.own;  // parallel block: a_l rows, then own residual rows
  // Parallel block: the O prologue, which waits for the attention output
  // anyway, also fetches the down projection's input and the next layer's
  // input and RMSNorm gains.  The down, QKV and gate/up prologues after it
  // then issue no global loads (theirs would complete behind the ring loads
  // the waves have just issued).
  const bool early = PAR && G <= 2 && p.lp.hb >= 0;  // (four query heads per KV head: too many registers)
  // pipelined phase order (set by the host only where early holds): the O
  // prologue of layer l stages layer l + 2's input, which layer l + 2 reads
  // after layer l + 1's phases
  const int pipe = p.lp.pipe;
  // x_{l+1+pipe} comes from the down projection of layer l + pipe - delay,
  // which has run before the O prologue of layer l only for delay > pipe;
  // otherwise each QKV polls its own input
  const bool stage_x = p.m.delay > pipe;
  float* const hbs = lds_dyn + (early ? p.lp.hb : 0);
  uint16_t* const gst = (uint16_t*)(lds_dyn + (early ? p.lp.gst : 0));
  int* wgrows = D.desc + kWaves * kWaveDesc;

  if (D.tid == 0) *abort_flag(D) = 0;
  // descriptors: every lane of a wave computes, lane 0 stores
  {
    int dsc[8], rows[2];
    const int kinds[5] = {PH_QKV, PH_O, PH_GU, PH_DOWN, PH_LM};
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      write_gemv_desc<G>(p, kinds[k], D.nwg, D.wg, D.wave, dsc, rows);
      if (D.lane == 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) D.desc[D.wave * kWaveDesc + 8 * k + i] = dsc[i];
        if (D.wave == 0) {
          wgrows[2 * k] = rows[0];
          wgrows[2 * k + 1] = rows[1];
        }
      }
    }
  }
  wg_sync();

  // cursor and ring (started at the top of every step)
  Cursor cur;
  cur.base = (uint64_t)(uintptr_t)p.W;
  cur.voff = 0;
  cur.stride = kChunkBytes;
  cur.rem = 0;
  cur.attn = 0;
  cur.kvh = 0;
  cur.seg = 0;
  cur.ph = 0;
  cur.nph = 0;
  cur.done = 1;
  cur.layer = 0;
  int slot = 0;

  int token = 0;

  for (int s = 0; s < p.n_steps; ++s) {
    const uint32_t epoch = p.epoch0 + (uint32_t)s;
    const int pos = p.pos0 + s;
    // this step's attention descriptor (read by the consumer and the cursor)
    int* adesc = D.desc + D.wave * kWaveDesc + kConsumerAttn;
    {
      int ad[12];
      write_attn_desc<G>(p, D.nwg, D.wg, D.wave, D.kpl, pos, ad);
#pragma unroll
      for (int i = 0; i < 12; ++i) adesc[i] = ad[i];
    }
    // restart the cursor on this step and fill the ring.  Every earlier ring
    // load has completed (the end-of-step polls waited for them), so the
    // slots can be reused in order from `slot`.
    __builtin_amdgcn_s_waitcnt(kWaitAllVm);
    cur.ph = 0;
    cur.nph = nphases(p, s);
    cur.done = 0;
    cursor_enter(D, cur);
#pragma unroll 1
    for (int i = 0; i < kDepth; ++i) cursor_issue(D, cur, ring_add(slot, i));

    trace_begin(D, s);
    // ---- input token and embedding ------------------------------------
    if (p.forced) {
      token = p.forced[s];
    } else if (s == 0) {
      token = p.first_from_state ? D.state[2] : 0;
    }
    if (token < 0 || token >= V) {
      if (D.tid == 0 && D.wg == 0) atomicCAS(&D.state[0], 0, (int)DEV_BAD_TOKEN);
      token = 0;
    }
    {
      // all loads first, then the conversions (see load_gains)
      const uint16_t* e = p.W + p.pl.embed + (uint64_t)token * d;
      uint16_t ev[kGainRegs];
      const int t = opaque(D.tid);
#pragma unroll
      for (int k = 0; k < kGainRegs; ++k) {
        const int i = t + k * kThreads;
        ev[k] = e[i < d ? i : 0];
      }
#pragma unroll
      for (int k = 0; k < kGainRegs; ++k) {
        const int i = t + k * kThreads;
        if (i < d) xraw[i] = hbits2f(ev[k]);
      }
    }
    wg_sync();
    // parallel block: this thread's RoPE factors for every layer's QKV
    // epilogue (the position and the workgroup's QKV rows are the same in
    // every layer), so that no QKV prologue loads them
    float2 rope_step = make_float2(1.f, 0.f);
    if (PAR) {
      const int r0 = wgrows[2 * 3], nr = wgrows[2 * 3 + 1];
      for (int t = D.tid; t < nr; t += kThreads) own[nr + t] = xraw[r0 + t];
      const int qr0 = wgrows[2 * gemv_index(PH_QKV)], qn = wgrows[2 * gemv_index(PH_QKV) + 1];
      const int rr = qr0 + 2 * D.tid;
      const bool mine = 2 * D.tid < qn && rr < qd + kvd;
      const int i = mine ? ((rr < qd ? rr : rr - qd) % hd) >> 1 : 0;
      rope_step = D.rope[(uint64_t)pos * (hd / 2) + i];
      wg_sync();
    }

    if ((p.debug_flags & DBG_WAIT_NEVER) && D.wg == 0) {
      // wait on a word that no one writes: exercises the bounded wait
      if (D.tid == 0) {
        u64 dummy;
        spin_word(D, D.LMP + 2 * D.nwg - 1, 0xFFFFFFFFu, &dummy);
      }
      wg_sync();
      if (aborted(D)) { __builtin_amdgcn_s_waitcnt(kWaitAllVm); return; }
    }

    const int nph = nphases(p, s);
    for (int ph = 0; ph < nph; ++ph) {
      const bool is_lm = ph == 5 * L;
      int kind = PH_LM, l = L;
      if (!is_lm) phase_at(pipe, PAR, L, ph, &kind, &l);
      const uint16_t* Wl = p.W + (uint64_t)(is_lm ? 0 : l) * p.pl.layer_stride;

      stamp(D, s, ph, 0);
      if (p.debug_flags & DBG_JITTER) jitter(D, epoch, ph);
      if (kind == PH_ATTN) {
        // ================= attention over the KV cache ==================
        float mrow[G], lrow[G], acc[G][8], q[G][8];
        const int nseg = rfl(adesc[10]);
        Owed owed{0, 0};
        // The query heads of every segment and the key and value at the
        // current position (all written by this step's QKV epilogue), polled
        // once by the whole workgroup into LDS: qkv[sg][G + 2][hd].  No wave
        // then waits on a remote word between or after its streams.
        float* qkv = lds_dyn + p.lp.attn_qkv;
        {
          const int per = (G + 2) * hd;
          const int g0 = rfl(adesc[0]), g1 = rfl(adesc[5]);
          for (int base = D.tid; base < nseg * per; base += kThreads * 8) {
            const u64* a[8];
            uint32_t mask = 0;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              const int i = base + k * kThreads;
              a[k] = D.Q;
              if (i < nseg * per) {
                const int sg = i / per, j = i % per, row = j / hd, dd = j % hd;
                const int g = sg ? g1 : g0;
                a[k] = row < G ? D.Q + (uint64_t)l * qd + (uint64_t)(g * G + row) * hd + dd
                               : (row == G ? D.KC : D.VC) + (uint64_t)l * kvd + (uint64_t)g * hd + dd;
                mask |= 1u << k;
              }
            }
            u64 v[8];
            if (!poll_addrs<8>(D, a, mask, epoch, v)) break;
#pragma unroll
            for (int k = 0; k < 8; ++k)
              if (mask & (1u << k)) qkv[base + k * kThreads] = ll_f(v[k]);
          }
        }
        wg_sync();
        if (aborted(D)) { __builtin_amdgcn_s_waitcnt(kWaitAllVm); return; }
        stamp(D, s, ph, 1);
        for (int sg = 0; sg < nseg; ++sg) {
          const int ka = rfl(adesc[5 * sg + 1]), kc = rfl(adesc[5 * sg + 2]), nst = rfl(adesc[5 * sg + 3]);
          const int has_pos = rfl(adesc[5 * sg + 4]);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            mrow[h] = -INFINITY;
            lrow[h] = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
          }
          // this lane's 8 query dims of every head in the group
          const float* qs = qkv + sg * (G + 2) * hd + D.dl * 8;
#pragma unroll
          for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) q[h][e] = qs[h * hd + e];
          attn_stream<G>(D, cur, slot, owed, nst, ka, kc, q, mrow, lrow, acc);
          if (has_pos) {
            // current key and value (fp16-rounded by the QKV epilogue)
            float kx[8], vx[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              kx[e] = qs[G * hd + e];
              vx[e] = qs[(G + 1) * hd + e];
            }
            const bool mine = D.lane < D.lpk;
#pragma unroll
            for (int h = 0; h < G; ++h) {
              float t = 0.f;
#pragma unroll
              for (int e = 0; e < 8; ++e) t = __builtin_fmaf(kx[e], q[h][e], t);
              t = group_sum(t, D.lpk, D.dl);
              if (mine) online_update(mrow[h], lrow[h], acc[h], t, vx);
            }
          }
          // merge this wave's key slots into slot 0 (lanes 0..lpk-1) as a
          // tree: with span s, slot j < s takes in slot j + s (when it
          // exists), for s = the largest power of two below kpl, then halves.
          // Every slot is counted exactly once.
          int span = 1;
          while (span * 2 < D.kpl) span *= 2;
          for (; span >= 1; span >>= 1) {
            const int src = (D.lane + span * D.lpk) & (kWave - 1);
            const bool take = D.kl < span && D.kl + span < D.kpl;
#pragma unroll
            for (int h = 0; h < G; ++h) {
              const float mo = __shfl(mrow[h], src);
              const float lo = __shfl(lrow[h], src);
              float ao[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) ao[e] = __shfl(acc[h][e], src);
              if (take) lse_merge(mrow[h], lrow[h], acc[h], mo, lo, ao);
            }
          }
          if (D.lane < D.lpk) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
              float* r = wrec + ((sg * kWaves + D.wave) * G + h) * (hd + 2);
              if (D.lane == 0) {
                r[0] = mrow[h];
                r[1] = lrow[h];
              }
#pragma unroll
              for (int e = 0; e < 8; ++e) r[2 + D.dl * 8 + e] = acc[h][e];
            }
          }
        }
        wg_sync();
        if (aborted(D)) { __builtin_amdgcn_s_waitcnt(kWaitAllVm); return; }
        // workgroup merge of the waves -> one record per segment
        for (int sg = 0; sg < nseg; ++sg) {
          u64* rec = D.REC + (((uint64_t)l * D.nwg + D.wg) * 2 + sg) * G * (hd + 2);
          for (int t = D.tid; t < G * hd; t += kThreads) {
            const int h = t / hd, dd = t % hd;
            float M = -INFINITY;
            for (int w = 0; w < kWaves; ++w) M = fmaxf(M, wrec[((sg * kWaves + w) * G + h) * (hd + 2)]);
            float Ls = 0.f, O = 0.f;
            for (int w = 0; w < kWaves; ++w) {
              const float* r = wrec + ((sg * kWaves + w) * G + h) * (hd + 2);
              const float a = r[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(r[0] - M);
              Ls += a * r[1];
              O += a * r[2 + dd];
            }
            if (dd == 0) {
              ll_storef(rec + h * (hd + 2) + 0, M, epoch);
              ll_storef(rec + h * (hd + 2) + 1, Ls, epoch);
            }
            ll_storef(rec + h * (hd + 2) + 2 + dd, O, epoch);
          }
        }
        stamp(D, s, ph, 2);
        // merger: the workgroup holding head g's last key combines the
        // records of every workgroup that met head g
        const int merge_g = rfl(adesc[11]);
        bool lone_merger = merge_g >= 0;
        if constexpr (G > 2) {
          // a merger of one query head (attn_mergers): head mh's words of
          // every record of the group, one weight per record, hd outputs
          lone_merger = merge_g >= 0 && (merge_g >> 16) == 0;
          if (merge_g >= 0 && (merge_g >> 16) > 0) {
            const int g = merge_g & 0xFFFF, mh = (merge_g >> 16) - 1;
            const int n_ctx = pos + 1;
            const int w_first = attn_owner(Hkv, n_ctx, D.nwg, g, 0);
            const int nrec = attn_owner(Hkv, n_ctx, D.nwg, g, n_ctx - 1) - w_first + 1;
            for (int r = D.tid; r < nrec; r += kThreads) {
              AttnSeg sgs[2];
              sgs[0] = AttnSeg{0, 0, 0};
              sgs[1] = AttnSeg{0, 0, 0};
              const int ns = attn_segments(Hkv, n_ctx, D.nwg, w_first + r, sgs);
              mlw[r * 8 + 7] = ns > 0 ? (float)((sgs[0].g == g) ? 0 : 1) : -1.f;
            }
            wg_sync();
            float* recs = wrec;  // the wave records are consumed already
            const int hw = hd + 2;
            merger_poll_wide<9>(D, l, w_first, nrec, G * hw, hw, mh * hw, hd, mlw, recs, epoch);
            wg_sync();
            if (aborted(D)) { __builtin_amdgcn_s_waitcnt(kWaitAllVm); return; }
            if (D.wave == 0) {
              float M = -INFINITY;
              for (int r = D.lane; r < nrec; r += kWave) M = fmaxf(M, recs[r * hw]);
              M = wave_max(M);
              float Ls = 0.f;
              for (int r = D.lane; r < nrec; r += kWave)
                Ls += (recs[r * hw] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(recs[r * hw] - M)) * recs[r * hw + 1];
              Ls = wave_sum(Ls);
              for (int r = D.lane; r < nrec; r += kWave)
                mlw[r * 8] = (recs[r * hw] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(recs[r * hw] - M)) / Ls;
            }
            wg_sync();
            for (int t = D.tid; t < hd; t += kThreads) {
              float o = 0.f;
#pragma unroll 4
              for (int r = 0; r < nrec; ++r) o += mlw[r * 8] * recs[r * hw + 2 + t];
              ll_storef(D.OB + (uint64_t)l * qd + (uint64_t)(g * G + mh) * hd + t, o, epoch);
            }
          }
        }
        if (lone_merger) {
          const int g = merge_g;
          const int n_ctx = pos + 1;
          const int w_first = attn_owner(Hkv, n_ctx, D.nwg, g, 0);
          const int nrec = D.wg - w_first + 1;
          // 1. which records exist: mlw[r*8 + 7] = segment of record r or -1
          for (int r = D.tid; r < nrec; r += kThreads) {
            AttnSeg sgs[2];
            sgs[0] = AttnSeg{0, 0, 0};
            sgs[1] = AttnSeg{0, 0, 0};
            const int ns = attn_segments(Hkv, n_ctx, D.nwg, w_first + r, sgs);
            mlw[r * 8 + 7] = ns > 0 ? (float)((sgs[0].g == g) ? 0 : 1) : -1.f;
          }
          wg_sync();
          // 2. one poll round: every word of every record into LDS
          //    (record r, head h at recs[(r*G + h)*(hd+2) ...])
          float* recs = wrec;  // the wave records are consumed already
          const int rw = G * (hd + 2);
          if constexpr (G > 2) {
            merger_poll_wide<17>(D, l, w_first, nrec, rw, rw, 0, hd, mlw, recs, epoch);
          } else {
          for (int base = D.tid; base < nrec * rw; base += kThreads * 8) {
            u64 vv[8];
            uint32_t mask = 0;
            const u64* addr[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              const int i = base + k * kThreads;
              addr[k] = D.REC;
              if (i < nrec * rw) {
                const int r = i / rw, off = i % rw;
                const int si = (int)mlw[r * 8 + 7];
                if (si >= 0) {
                  addr[k] = D.REC + (((uint64_t)l * D.nwg + w_first + r) * 2 + si) * rw + off;
                  mask |= 1u << k;
                }
              }
            }
#pragma unroll
            for (int k = 0; k < 8; ++k)
              if (mask & (1u << k)) vv[k] = ll_load(addr[k]);
            const uint64_t t0 = wall_clock64();
            for (int it = 0;; ++it) {
              uint32_t stale = 0;
#pragma unroll
              for (int k = 0; k < 8; ++k)
                if ((mask & (1u << k)) && ll_epoch(vv[k]) != epoch) stale |= 1u << k;
              if (!stale) break;
              if ((it & 15) == 15) {
                if (abort_seen(D)) break;
                if (__hip_atomic_load(&D.state[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
                  set_abort(D);
                  break;
                }
                if (wall_clock64() - t0 > D.p->timeout_ticks) {
                  raise_status(D, DEV_TIMEOUT);
                  break;
                }
              }
              __builtin_amdgcn_s_sleep(1);
#pragma unroll
              for (int k = 0; k < 8; ++k)
                if (stale & (1u << k)) vv[k] = ll_load(addr[k]);
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              const int i = base + k * kThreads;
              if (i < nrec * rw) {
                const int off = i % rw;
                float v = 0.f;
                if (mask & (1u << k)) {
                  v = ll_f(vv[k]);
                } else if (off % (hd + 2) == 0) {
                  v = -INFINITY;  // missing record: empty
                }
                recs[i] = v;
              }
            }
          }
          }
          wg_sync();
          if (aborted(D)) { __builtin_amdgcn_s_waitcnt(kWaitAllVm); return; }
          // 3. combine: o = sum_r c_r O_r with c_r = exp2(m_r - M) / L and
          //    L = sum_r exp2(m_r - M) l_r.  First one wave per query head
          //    computes every record's weight (lanes over records), then
          //    every output sums its column with independent LDS reads.
          if (D.wave < G) {
            const int h = D.wave;
            float M = -INFINITY;
            for (int r = D.lane; r < nrec; r += kWave) M = fmaxf(M, recs[(r * G + h) * (hd + 2)]);
            M = wave_max(M);
            float Ls = 0.f;
            for (int r = D.lane; r < nrec; r += kWave) {
              const float* rr = recs + (r * G + h) * (hd + 2);
              Ls += (rr[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(rr[0] - M)) * rr[1];
            }
            Ls = wave_sum(Ls);
            for (int r = D.lane; r < nrec; r += kWave) {
              const float* rr = recs + (r * G + h) * (hd + 2);
              mlw[r * 8 + h] = (rr[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(rr[0] - M)) / Ls;
            }
          }
          wg_sync();
          for (int t = D.tid; t < G * hd; t += kThreads) {
            const int h = t / hd, dd = t % hd;
            float o = 0.f;
#pragma unroll 4
            for (int r = 0; r < nrec; ++r) o += mlw[r * 8 + h] * recs[(r * G + h) * (hd + 2) + 2 + dd];
            ll_storef(D.OB + (uint64_t)l * qd + (uint64_t)(g * G + h) * hd + dd, o, epoch);
          }
        }
        // the records (and a merger's output) are out: now the deferred loads
        issue_owed(D, cur, owed);
        wg_sync();
        if (aborted(D)) { __builtin_amdgcn_s_waitcnt(kWaitAllVm); return; }
        stamp(D, s, ph, 3);
        continue;
      }

      // ===================== GEMV phases =====================
      const int gi = gemv_index(kind);
      const int r0 = rfl(wgrows[2 * gi]), nrows = rfl(wgrows[2 * gi + 1]);
      // prologue: the input vector
      uint16_t gr[kGainRegs];
      float2 rope_cs = make_float2(1.f, 0.f);
      // gains (and, with a delay that publishes x in time, the input x)
      // fetched by an O prologue
      const bool staged = early && l > pipe && !is_lm;
      const bool staged_x = staged && stage_x;
      if (kind == PH_QKV) {
        if (staged) {
          stashed_gains(D, gst, gr);
        } else {
          load_gains(D, Wl + p.pl.attn_norm, gr);
        }
        // this thread's RoPE factors for the epilogue, fetched ahead too
        // (unconditionally, from a clamped index: see load_gains)
        if (PAR) {
          rope_cs = rope_step;
        } else {
          const int rr = r0 + 2 * D.tid;
          const bool mine = 2 * D.tid < nrows && rr < qd + kvd;
          const int i = mine ? ((rr < qd ? rr : rr - qd) % hd) >> 1 : 0;
          rope_cs = D.rope[(uint64_t)pos * (hd / 2) + i];
        }
        asm volatile("" ::: "memory");
        if (!staged_x && (PAR ? (l > p.m.delay) : (l > 0))) {
          const int xi = PAR ? l : 2 * l;
          poll_to_lds<false>(D, D.X + (uint64_t)xi * d, xraw, d, epoch);
          wg_sync();
          if (aborted(D)) { __builtin_amdgcn_s_waitcnt(kWaitAllVm); return; }
        }
        if (early) {
          // gate/up's input too, into the down input's area (idle until O)
          uint16_t gg[kGainRegs];
          if (staged) {
            stashed_gains(D, gst + gains_pad(d), gg);
          } else {
            load_gains(D, Wl + p.pl.mlp_norm, gg);
          }
          gain2_to_xs(D, xraw, gr, xs, gg, hbs);
        } else {
          if (PAR) {
            rmsnorm_to_xs(D, xraw, gr, xs);
          } else {
            gain_to_xs(D, xraw, gr, xs);
          }
        }
      } else if (kind == PH_GU && early) {
        // input prepared by the QKV prologue
      } else if (kind == PH_GU) {
        if (staged) {
          stashed_gains(D, gst + gains_pad(d), gr);
        } else {
          load_gains(D, Wl + p.pl.mlp_norm, gr);
        }
        if (!PAR) {
          poll_to_lds<false>(D, D.X + (uint64_t)(2 * l + 1) * d, xraw, d, epoch);
          wg_sync();
          if (aborted(D)) { __builtin_amdgcn_s_waitcnt(kWaitAllVm); return; }
        }
        if (PAR) {
          rmsnorm_to_xs(D, xraw, gr, xs);
        } else {
          gain_to_xs(D, xraw, gr, xs);
        }
      } else if (kind == PH_O) {
        if (early) {
          // the input of the next QKV of a layer above 0 (layer l + 1, or
          // l + 2 in the pipelined order)
          const int ln = l + 1 + pipe;
          const bool next = ln < L;
          if (next) {
            copy_halves(D, Wl + (uint64_t)(1 + pipe) * p.pl.layer_stride + p.pl.attn_norm, gst, d);
            copy_halves(D, Wl + (uint64_t)(1 + pipe) * p.pl.layer_stride + p.pl.mlp_norm, gst + gains_pad(d), d);
          }
          const bool want_hb = rfl(wgrows[2 * gemv_index(PH_DOWN) + 1]) > 0;
          const bool want_x = stage_x && next && ln > p.m.delay;
          // two round trips: down's input, then the next x and the
          // attention output together (when they fit the batches)
          const PollSeg s1[3] = {{D.HB + (uint64_t)l * F, hbs, want_hb ? F : 0, 1},
                                 {D.HB, hbs, 0, 1},
                                 {D.HB, hbs, 0, 1}};
          const PollSeg s2[3] = {{D.X + (uint64_t)ln * d, xraw, want_x ? d : 0, 0},
                                 {D.OB + (uint64_t)l * qd, xs, qd, 1},
                                 {D.OB, xs, 0, 1}};
          if (s1[0].n <= kMultiPoll1 * kThreads) {
            (void)poll_multi<kMultiPoll1>(D, s1, epoch);
          } else {
            poll_to_lds<true>(D, s1[0].src, hbs, F, epoch);
          }
          if (G <= 2 && s2[0].n + s2[1].n <= kMultiPoll2 * kThreads) {
            (void)poll_multi<kMultiPoll2>(D, s2, epoch);
          } else {
            if (want_x) poll_to_lds<false>(D, s2[0].src, xraw, d, epoch);
            poll_to_lds<true>(D, s2[1].src, xs, qd, epoch);
          }
          if (want_hb) zero_tail(D, hbs, F);
        } else {
          poll_to_lds<true>(D, D.OB + (uint64_t)l * qd, xs, qd, epoch);
        }
        zero_tail(D, xs, qd);
        // (loads complete in order: the gain copies, issued before the polls,
        // have landed; the wait only makes it explicit)
        if (early) __builtin_amdgcn_s_waitcnt(kWaitAllVm);
      } else if (kind == PH_DOWN) {
        if (!early) {
          // one batch of loads when it fits (a second batch would be issued
          // only once the first is complete: one more round trip)
          const PollSeg sd[3] = {{D.HB + (uint64_t)l * F, xs, F, 1}, {D.HB, xs, 0, 1}, {D.HB, xs, 0, 1}};
          if (!PAR && G == 1 && F <= kMultiPoll1 * kThreads) {  // (more heads per KV head: too many registers)
            (void)poll_multi<kMultiPoll1>(D, sd, epoch);
          } else {
            poll_to_lds<true>(D, D.HB + (uint64_t)l * F, xs, F, epoch);
          }
          zero_tail(D, xs, F);
        }
      } else {  // LM
        load_gains(D, p.W + p.pl.final_norm, gr);
        poll_to_lds<false>(D, D.X + (uint64_t)(2 * L) * d, xraw, d, epoch);
        wg_sync();
        if (aborted(D)) { __builtin_amdgcn_s_waitcnt(kWaitAllVm); return; }
        gain_to_xs(D, xraw, gr, xs);
      }
      for (int i = D.tid; i < nrows * kWaves; i += kThreads) part[i] = 0.f;
      wg_sync();
      if (aborted(D)) { __builtin_amdgcn_s_waitcnt(kWaitAllVm); return; }
      stamp(D, s, ph, 1);

      {
        const int* gd = D.desc + D.wave * kWaveDesc + 8 * gi;
        const float* gin = (early && (kind == PH_DOWN || kind == PH_GU)) ? hbs : xs;
        gemv_stream(D, cur, slot, gin, part, rfl(gd[2]), rfl(gd[3]), rfl(gd[4]), rfl(gd[5]));
      }
      stamp(D, s, ph, 2);
      wg_sync();

      // epilogue
      // the deferred RMSNorm scale (gain_to_xs / gain2_to_xs); the parallel
      // block's gate/up reads the sums its QKV prologue left
      const bool deferred = kind == PH_LM || ((kind == PH_QKV || kind == PH_GU) && (!PAR || early));
      const float ninv = deferred ? rms_inv(D) : 1.f;
      if (kind == PH_QKV) {
        const float qscale = 1.4426950408889634f / sqrtf((float)hd);
        const float2* rp = D.rope + (uint64_t)pos * (hd / 2);
        for (int t = D.tid; t < nrows / 2; t += kThreads) {
          float y0 = 0.f, y1 = 0.f;
#pragma unroll
          for (int w = 0; w < kWaves; ++w) {
            y0 += part[(2 * t) * kWaves + w];
            y1 += part[(2 * t + 1) * kWaves + w];
          }
          y0 *= ninv;
          y1 *= ninv;
          const int rr = r0 + 2 * t;
          if (rr < qd + kvd) {
            const bool isq = rr < qd;
            const int base = isq ? 0 : qd;
            const int head = (rr - base) / hd;
            const int i = ((rr - base) % hd) >> 1;
            const float2 cs = t == D.tid ? rope_cs : rp[i];
            const float a = y0 * cs.x - y1 * cs.y;
            const float b = y0 * cs.y + y1 * cs.x;
            if (isq) {
              u64* qp = D.Q + (uint64_t)l * qd + (uint64_t)head * hd;
              ll_storef(qp + i, a * qscale, epoch);
              ll_storef(qp + i + hd / 2, b * qscale, epoch);
            } else {
              const __half ah = __float2half_rn(a), bh = __float2half_rn(b);
              uint16_t* kc = p.kv + kv_offset(p.m, l, 0, head) + (uint64_t)pos * hd;
              kc[i] = __half_as_ushort(ah);
              kc[i + hd / 2] = __half_as_ushort(bh);
              u64* kp = D.KC + (uint64_t)l * kvd + (uint64_t)head * hd;
              ll_storef(kp + i, __half2float(ah), epoch);
              ll_storef(kp + i + hd / 2, __half2float(bh), epoch);
            }
          } else {
            const int jv = rr - qd - kvd;
            const int head = jv / hd, dd = jv % hd;
            const __half ah = __float2half_rn(y0), bh = __float2half_rn(y1);
            uint16_t* vc = p.kv + kv_offset(p.m, l, 1, head) + (uint64_t)pos * hd;
            vc[dd] = __half_as_ushort(ah);
            vc[dd + 1] = __half_as_ushort(bh);
            u64* vp = D.VC + (uint64_t)l * kvd + (uint64_t)head * hd;
            ll_storef(vp + dd, __half2float(ah), epoch);
            ll_storef(vp + dd + 1, __half2float(bh), epoch);
          }
        }
      } else if (kind == PH_GU) {
        for (int t = D.tid; t < nrows / 2; t += kThreads) {
          float y0 = 0.f, y1 = 0.f;
#pragma unroll
          for (int w = 0; w < kWaves; ++w) {
            y0 += part[(2 * t) * kWaves + w];
            y1 += part[(2 * t + 1) * kWaves + w];
          }
          y0 *= ninv;
          y1 *= ninv;
          const float hval = y0 / (1.0f + expf(-y0)) * y1;
          ll_storef(D.HB + (uint64_t)l * F + (r0 >> 1) + t, hval, epoch);
        }
      } else if (kind == PH_O) {
        for (int t = D.tid; t < nrows; t += kThreads) {
          float y = 0.f;
#pragma unroll
          for (int w = 0; w < kWaves; ++w) y += part[t * kWaves + w];
          if (PAR) {
            own[t] = y;  // a_l for the rows this workgroup owns
          } else {
            ll_storef(D.X + (uint64_t)(2 * l + 1) * d + r0 + t, xraw[r0 + t] + y, epoch);
          }
        }
      } else if (kind == PH_DOWN) {
        for (int t = D.tid; t < nrows; t += kThreads) {
          float y = 0.f;
#pragma unroll
          for (int w = 0; w < kWaves; ++w) y += part[t * kWaves + w];
          if (PAR) {
            // P_l = a_l + m_l reaches the residual of layer l + delay + 1
            const float xn = own[nrows + t] + (own[t] + y);
            own[nrows + t] = xn;
            const int k = l + p.m.delay + 1;
            if (l == L - 1) {
              ll_storef(D.X + (uint64_t)(2 * L) * d + r0 + t, xn, epoch);
            } else if (k <= L - 1) {
              ll_storef(D.X + (uint64_t)k * d + r0 + t, xn, epoch);
            }
          } else {
            const int xo = (l == L - 1) ? 2 * L : 2 * l + 2;
            ll_storef(D.X + (uint64_t)xo * d + r0 + t, xraw[r0 + t] + y, epoch);
          }
        }
      } else {  // LM: logits and this workgroup's argmax
        const int out_step = p.lm_mode == 1 ? 0 : s;
        float my_val = -INFINITY;
        int my_idx = 0x7FFFFFFF;
        for (int t = D.tid; t < nrows; t += kThreads) {
          float y = 0.f;
#pragma unroll
          for (int w = 0; w < kWaves; ++w) y += part[t * kWaves + w];
          y *= ninv;
          const int row = r0 + t;
          if (p.logits) p.logits[(uint64_t)out_step * V + row] = y;
          // sampling: the Gumbel-max draw over logits / T
          const float sc = p.sample ? y * p.inv_temp + gumbel(philox_w0((uint32_t)row, (uint32_t)pos, p.seed_lo, p.seed_hi))
                                    : y;
          if (argmax_better(sc, row, my_val, my_idx)) {
            my_val = sc;
            my_idx = row;
          }
        }
        wave_argmax(my_val, my_idx);
        if (D.lane == 0) {
          D.sh->lmv[D.wave] = my_val;
          D.sh->lmi[D.wave] = my_idx;
        }
      }
      wg_sync();
      stamp(D, s, ph, 3);
    }  // phases

    // ---- end of step: release the KV writes, publish, gather ------------
    const int tph = 5 * 64 + 1;
    stamp(D, s, tph, 0);
    const bool lm = lm_active(p, s);
    if (p.debug_flags & DBG_JITTER) jitter(D, epoch, tph);
    // every thread's KV-cache stores have reached the L2 before thread 0's
    // release fence writes the L2 back (one write-back per workgroup)
    __builtin_amdgcn_s_waitcnt(kWaitAllVm);
    wg_sync();
    if (D.tid == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      float bv = -INFINITY;
      int bi = 0x7FFFFFFF;
      if (lm) {
        bv = D.sh->lmv[0];
        bi = D.sh->lmi[0];
        for (int w = 1; w < kWaves; ++w) {
          const float ov = D.sh->lmv[w];
          const int oi = D.sh->lmi[w];
          if (argmax_better(ov, oi, bv, bi)) {
            bv = ov;
            bi = oi;
          }
        }
      }
      ll_storef(D.LMP + 2 * D.wg, bv, epoch);
      ll_store(D.LMP + 2 * D.wg + 1, (uint32_t)bi, epoch);
    }
    // every workgroup reads every partial and takes the same decision: each
    // thread keeps the best of the partials it polled, then each wave's best
    // goes to LDS
    {
      float bv = -INFINITY;
      int bi = 0x7FFFFFFF;
      for (int t = D.tid; t < D.nwg; t += kThreads) {
        u64 ab[2];
        poll_words<2>(D, D.LMP + 2 * t, 1, 3u, epoch, ab);
        const float ov = ll_f(ab[0]);
        const int oi = (int)(uint32_t)ab[1];
        if (argmax_better(ov, oi, bv, bi)) {
          bv = ov;
          bi = oi;
        }
      }
      wave_argmax(bv, bi);
      if (D.lane == 0) {
        D.sh->tokv[D.wave] = bv;
        D.sh->toki[D.wave] = bi;
      }
    }
    wg_sync();
    // every workgroup's release is now observed: one acquire (L1 and L2
    // invalidate) before this workgroup reads KV rows of the next step
    if (D.tid == 0) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      __builtin_amdgcn_s_waitcnt(kWaitAllVm);
    }
    wg_sync();
    if (aborted(D)) { __builtin_amdgcn_s_waitcnt(kWaitAllVm); return; }
    stamp(D, s, tph, 1);
    if (lm) {
      // every thread reduces the eight wave results the same way
      float bv = D.sh->tokv[0];
      int bi = D.sh->toki[0];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) {
        const float ov = D.sh->tokv[w];
        const int oi = D.sh->toki[w];
        if (argmax_better(ov, oi, bv, bi)) {
          bv = ov;
          bi = oi;
        }
      }
      token = rfl(bi);
      if (D.wg == 0 && D.tid == 0) {
        if (p.out) p.out[p.lm_mode == 1 ? 0 : s] = token;
        D.state[2] = token;
      }
    }
    wg_sync();
    trace_end(D, s);
  }  // steps
  __builtin_amdgcn_s_waitcnt(kWaitAllVm);  // no ring DMA may outlive the workgroup
}

// fill with zeros (a graph-capturable replacement for a memset)
__global__ void kie_zero_kernel(uint4* p, uint64_t n16) {
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (uint64_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

}  // namespace KIE_RING_NS
}  // namespace kie

// ---------------------------------------------------------------------------
// host-side launch helpers (called by the C-ABI in kie_api.cpp)
// ---------------------------------------------------------------------------
// one kernel per (query heads per KV head, block kind): the sequential and
// the parallel block are separate instantiations, so neither carries the
// other's branches
static const void* kie_kernel_for(int G, int parallel) {
  switch (G * 2 + (parallel ? 1 : 0)) {
    case 2: return (const void*)&kie::KIE_RING_NS::kie_monokernel<1, false>;
    case 3: return (const void*)&kie::KIE_RING_NS::kie_monokernel<1, true>;
    case 4: return (const void*)&kie::KIE_RING_NS::kie_monokernel<2, false>;
    case 5: return (const void*)&kie::KIE_RING_NS::kie_monokernel<2, true>;
    case 8: return (const void*)&kie::KIE_RING_NS::kie_monokernel<4, false>;
    case 9: return (const void*)&kie::KIE_RING_NS::kie_monokernel<4, true>;
    default: return nullptr;
  }
}

extern "C" hipError_t KIE_RING_ENTRY(kie_internal_launch)(const kie::KParams* kp, int nwg, size_t lds_bytes,
                                                          hipStream_t stream) {
  const void* fn = kie_kernel_for(kp->m.G, kp->m.parallel);
  if (!fn) return hipErrorInvalidValue;
  (void)lds_bytes;  // all LDS is static
  void* args[] = {(void*)kp};
  return hipLaunchCooperativeKernel(fn, dim3(nwg), dim3(kie::kThreads), args, 0, stream);
}

extern "C" hipError_t KIE_RING_ENTRY(kie_internal_zero)(void* p, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  if (((uintptr_t)p & 15) || (bytes & 15)) return hipErrorInvalidValue;
  const uint64_t n16 = bytes / 16;
  const uint64_t want = (n16 + 255) / 256;
  const int blocks = (int)(want < 4096 ? want : 4096);
  hipLaunchKernelGGL(kie::KIE_RING_NS::kie_zero_kernel, dim3(blocks), dim3(256), 0, stream, (uint4*)p, n16);
  return hipGetLastError();
}

extern "C" hipError_t KIE_RING_ENTRY(kie_internal_occupancy)(int G, int parallel, size_t lds_bytes,
                                                             int* blocks_per_cu) {
  const void* fn = kie_kernel_for(G, parallel);
  if (!fn) return hipErrorInvalidValue;
  (void)lds_bytes;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, fn, kie::kThreads, 0);
}
