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
//    KV cache) through a ring of kDepth 16-byte-per-lane registers; the load
//    cursor runs ahead of the consumer across phase boundaries, so weight
//    bytes keep flowing while a wave waits for the activation it needs;
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

namespace kie {

typedef unsigned long long u64;
constexpr int kDepth = kRingDepth;  // 1-KB wave units in flight per wave (LDS ring slots)
// s_waitcnt immediate that waits until at most kDepth-1 vector memory
// operations are outstanding (expcnt and lgkmcnt left at their maximum)
constexpr int kWaitRing = ((kDepth - 1) & 15) | (((kDepth - 1) >> 4) << 14) | (7 << 4) | (15 << 8);
constexpr int kWaitAllVm = (7 << 4) | (15 << 8);
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
// sum over groups of `lpk` consecutive lanes; every lane of a group gets it
KIE_DI float group_sum(float v, int lpk) {
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
  const int lane = threadIdx.x & 63;
  const int base = lane - lane % lpk;
  float s = 0.f;
  for (int j = 0; j < lpk; ++j) s += __shfl(v, base + j);
  return s;
}

KIE_DI float h2f_lo(uint32_t u) { return __half2float(__ushort_as_half((unsigned short)(u & 0xFFFF))); }
KIE_DI float h2f_hi(uint32_t u) { return __half2float(__ushort_as_half((unsigned short)(u >> 16))); }
KIE_DI float hbits2f(uint16_t u) { return __half2float(__ushort_as_half(u)); }

// swizzled position of element k of a GEMV input vector in LDS: inside each
// 512-element block the first 4 of every lane's 8 elements are contiguous
// across lanes, then the last 4, so each 16-byte LDS read is conflict-free
KIE_DI int xs_pos(int k) {
  const int b = k >> 9, e = k & 511;
  return (b << 9) + (((e >> 2) & 1) << 8) + ((e >> 3) << 2) + (e & 3);
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
  int token;
  int pad[2];
  float redf[kWaves];
  float lmv[kWaves];
  int lmi[kWaves];
};

struct Dev {
  const KParams* p;
  int wg, nwg, wave, lane, tid;
  Shared* sh;
  int* desc;
  uint4* ring;  // this wave's kDepth x 1 KB LDS ring
  int32_t* state;
  u64 *X, *Q, *KC, *VC, *REC, *OB, *HB, *LMP;
  const float2* rope;
  int lpk, kpl, kl, dl, lane_active;
};

KIE_DI void raise_status(const Dev& D, int code) {
  atomicCAS(&D.state[0], 0, code);
  __hip_atomic_store(&D.state[1], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  D.sh->abort = 1;
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
      if (*(volatile int*)&D.sh->abort) return false;
      if (__hip_atomic_load(&D.state[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
        D.sh->abort = 1;
        return false;
      }
      if (wall_clock64() - t0 > D.p->timeout_ticks) {
        raise_status(D, DEV_TIMEOUT);
        return false;
      }
    }
  }
}

// phase trace stamp (thread 0 of the workgroup only)
KIE_DI void stamp(const Dev& D, int s, int ph, int k) {
  const KParams& p = *D.p;
  if (p.trace && s < p.trace_steps && D.tid == 0)
    p.trace[(((uint64_t)s * kTracePhases + ph) * D.nwg + D.wg) * 4 + k] = wall_clock64();
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
      if (*(volatile int*)&D.sh->abort) return false;
      if (__hip_atomic_load(&D.state[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
        D.sh->abort = 1;
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

// the workgroup polls words [0, n) of src into dst (swizzled for GEMV input)
template <bool SWZ>
KIE_DI void poll_to_lds(const Dev& D, const u64* src, float* dst, int n, uint32_t epoch) {
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
      if (i < n) dst[SWZ ? xs_pos(i) : i] = ll_f(v[k]);
    }
  }
}

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
KIE_DI void write_gemv_desc(const KParams& p, int kind, int nwg, int wg, int wave, int* dsc, int* wgrows) {
  const GemvShape sh = gemv_shape(p.m, kind);
  int r0, r1, u0, u1;
  gemv_rows(p.m, kind, nwg, wg, &r0, &r1);
  gemv_wave_units(r1 - r0, sh.K, wave, &u0, &u1);
  const int nb = blocks_per_row(sh.K);
  const uint64_t off = matrix_offset(p, kind) + (uint64_t)(r0 + u0 / nb) * (uint64_t)sh.K;
  dsc[0] = (int)(uint32_t)off;
  dsc[1] = (int)(uint32_t)(off >> 32);
  dsc[2] = u0 % nb;
  dsc[3] = u1 - u0;
  dsc[4] = nb;
  dsc[5] = sh.K / 8;
  dsc[6] = u0 / nb;
  dsc[7] = 0;
  if (wave == 0) {
    wgrows[0] = r0;
    wgrows[1] = r1 - r0;
  }
}

// one wave's attention work at position pos -> 12-int descriptor
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
      split(seg[s].tb - seg[s].ta, kWaves, wave, &wa, &wb);
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
  dsc[10] = nseg;
  dsc[11] = merge_g;
}

// ---------------------------------------------------------------------------
// the load cursor: walks this wave's unit sequence (weights and KV rows) over
// the whole launch and issues exactly one 16-byte-per-lane load per call
// ---------------------------------------------------------------------------
struct Cursor {
  int s, ph, nph, rem, kind, done;
  const uint4* rowp;  // gemv: current row
  int b, nb, K8;
  int st, kvh, ka, kc, nst;  // attention: current segment
  const uint16_t* kb;
  const uint16_t* vb;
  int seg1, l;  // attention: segment 1 still to come; layer
};

KIE_DI void cursor_enter(const Dev& D, Cursor& c) {
  const KParams& p = *D.p;
  const int lmph = 5 * p.m.L;
  const int kind = c.ph == lmph ? PH_LM : phase_kind(p.m.parallel, c.ph % 5);
  const int l = c.ph == lmph ? 0 : c.ph / 5;
  c.kind = kind;
  c.l = l;
  if (kind == PH_ATTN) {
    const int* a = D.desc + D.wave * kWaveDesc + kConsumerAttn;
    const int nst0 = a[3], nst1 = a[8];
    const bool first = nst0 > 0;
    const int g = first ? a[0] : a[5];
    c.st = 0;
    c.kvh = 0;
    c.rem = 2 * (nst0 + nst1);
    c.ka = first ? a[1] : a[6];
    c.kc = first ? a[2] : a[7];
    c.nst = first ? nst0 : nst1;
    c.seg1 = first && nst1 > 0;
    c.kb = p.kv + kv_offset(p.m, l, 0, g);
    c.vb = p.kv + kv_offset(p.m, l, 1, g);
    return;
  }
  const int* g = D.desc + D.wave * kWaveDesc + 8 * gemv_index(kind);
  const uint64_t off = (uint64_t)(uint32_t)g[0] | ((uint64_t)(uint32_t)g[1] << 32);
  c.rowp = (const uint4*)(p.W + (kind == PH_LM ? 0 : (uint64_t)l * p.pl.layer_stride) + off);
  c.b = g[2];
  c.rem = g[3];
  c.nb = g[4];
  c.K8 = g[5];
}

// The cursor never crosses into the next step by itself: the next step reads
// KV-cache rows written during this step, which are only visible after the
// end-of-step acquire.  At the end of its step it issues harmless loads until
// the consumer restarts it (cursor_restart) after that acquire.
KIE_DI void cursor_advance(const Dev& D, Cursor& c) {
  while (c.rem == 0 && !c.done) {
    if (++c.ph >= c.nph) {
      c.done = 1;
      break;
    }
    cursor_enter(D, c);
  }
}

// issue the next unit of the sequence into ring slot `slot` (one DMA per call)
KIE_DI void cursor_issue(const Dev& D, Cursor& c, int slot) {
  const KParams& p = *D.p;
  if (c.rem == 0) cursor_advance(D, c);
  // A lane with nothing to load reads the first packed kilobyte, which holds
  // finite fp16 values: its GEMV input element is zero and its attention key
  // is masked to probability 0, so it contributes exactly nothing.
  const uint4* a = (const uint4*)p.W + D.lane;
  if (!c.done) {
    if (c.kind == PH_ATTN) {
      const int key = c.ka + c.st * D.kpl + D.kl;
      if (D.lane_active && key < c.kc) a = (const uint4*)((c.kvh ? c.vb : c.kb) + (uint64_t)key * p.m.hd) + D.dl;
      if (c.kvh) {
        if (++c.st == c.nst && c.seg1) {
          const int* s1 = D.desc + D.wave * kWaveDesc + kConsumerAttn + 5;
          c.seg1 = 0;
          c.st = 0;
          c.ka = s1[1];
          c.kc = s1[2];
          c.nst = s1[3];
          c.kb = p.kv + kv_offset(p.m, c.l, 0, s1[0]);
          c.vb = p.kv + kv_offset(p.m, c.l, 1, s1[0]);
        }
      }
      c.kvh ^= 1;
    } else {
      const int sg = c.b * kBlock8 + D.lane;
      if (sg < c.K8) a = c.rowp + sg;  // the input tail of xs is zero for the others
      if (++c.b == c.nb) {
        c.b = 0;
        c.rowp += c.K8;
      }
    }
    --c.rem;
  }
  // 16 bytes per lane straight into LDS: lane i lands at slot + 16 i
  __builtin_amdgcn_global_load_lds((const void*)a, (__attribute__((address_space(3))) void*)(D.ring + slot * kWave),
                                   16, 0, 2 /* nt */);
}

// read this lane's 16 bytes of ring slots.  The reads are written as asm and
// wait for themselves, so the compiler neither sees an LDS access that the
// ring DMAs could alias nor leaves an output register in flight.
KIE_DI uint32_t ring_addr(const Dev& D, int slot) {
  return (uint32_t)(uintptr_t)(D.ring + slot * kWave + D.lane);
}
KIE_DI uint4 ring_read(const Dev& D, int slot) {
  uint4 x;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(x) : "v"(ring_addr(D, slot)) : "memory");
  return x;
}
KIE_DI void ring_read4(const Dev& D, int s0, int s1, int s2, int s3, uint4& x0, uint4& x1, uint4& x2, uint4& x3) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3)
      : "v"(ring_addr(D, s0)), "v"(ring_addr(D, s1)), "v"(ring_addr(D, s2)), "v"(ring_addr(D, s3))
      : "memory");
}

KIE_DI int ring_next(int s) { return s + 1 == kDepth ? 0 : s + 1; }

// ---------------------------------------------------------------------------
// the ring: consume the next n units.  Exactly one DMA is issued per unit
// consumed, so when units c..c+3 are read the kDepth-4 younger DMAs may stay
// in flight (vector memory reads complete in order).  Units are taken four at
// a time so that one LDS round trip serves four of them.
// ---------------------------------------------------------------------------
constexpr int kWaitRing4 = ((kDepth - 4) & 15) | (((kDepth - 4) >> 4) << 14) | (7 << 4) | (15 << 8);

template <class F>
KIE_DI void run_units(const Dev& D, Cursor& cur, int& slot, int n, F& consume) {
  int j = 0;
  for (; j + 4 <= n; j += 4) {
    __builtin_amdgcn_s_waitcnt(kWaitRing4);
    const int s0 = slot, s1 = ring_next(s0), s2 = ring_next(s1), s3 = ring_next(s2);
    uint4 x0, x1, x2, x3;
    ring_read4(D, s0, s1, s2, s3, x0, x1, x2, x3);
    cursor_issue(D, cur, s0);
    cursor_issue(D, cur, s1);
    cursor_issue(D, cur, s2);
    cursor_issue(D, cur, s3);
    slot = ring_next(s3);
    consume(x0, j, false);
    consume(x1, j + 1, false);
    consume(x2, j + 2, false);
    consume(x3, j + 3, j + 3 == n - 1);
  }
  for (; j < n; ++j) {
    __builtin_amdgcn_s_waitcnt(kWaitRing);
    const uint4 x = ring_read(D, slot);
    cursor_issue(D, cur, slot);
    slot = ring_next(slot);
    consume(x, j, j == n - 1);
  }
}

// ---------------------------------------------------------------------------
// prologue helpers
// ---------------------------------------------------------------------------
// xraw -> xs = g * x / sqrt(mean(x^2) + eps), swizzled, zero tail to nb*512
KIE_DI void rmsnorm_to_xs(const Dev& D, const float* xraw, const uint16_t* g, float* xs) {
  const KParams& p = *D.p;
  const int d = p.m.d;
  float ss = 0.f;
  for (int i = D.tid; i < d; i += kThreads) ss += xraw[i] * xraw[i];
  ss = wave_sum(ss);
  if (D.lane == 0) D.sh->redf[D.wave] = ss;
  wg_sync();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) tot += D.sh->redf[w];
  const float inv = 1.0f / sqrtf(tot / (float)d + p.m.eps);
  const int padded = blocks_per_row(d) * kBlock;
  for (int i = D.tid; i < padded; i += kThreads) {
    float v = 0.f;
    if (i < d) v = xraw[i] * inv * hbits2f(g[i]);
    xs[xs_pos(i)] = v;
  }
}

KIE_DI void zero_tail(const Dev& D, float* xs, int K) {
  const int padded = blocks_per_row(K) * kBlock;
  for (int i = K + D.tid; i < padded; i += kThreads) xs[xs_pos(i)] = 0.f;
}

// one GEMV phase's consumer: dot a 512-column block with the LDS input and
// write one partial row sum per (row, wave)
struct GemvConsume {
  const float4* xs4;
  float* part;
  int r, b, nb, lane, wave;
  float acc;
  KIE_DI void operator()(const uint4 x, int, bool last) {
    const float4 xa = xs4[b * 128 + lane];
    const float4 xb = xs4[b * 128 + 64 + lane];
    float t = acc;
    t = __builtin_fmaf(h2f_lo(x.x), xa.x, t);
    t = __builtin_fmaf(h2f_hi(x.x), xa.y, t);
    t = __builtin_fmaf(h2f_lo(x.y), xa.z, t);
    t = __builtin_fmaf(h2f_hi(x.y), xa.w, t);
    t = __builtin_fmaf(h2f_lo(x.z), xb.x, t);
    t = __builtin_fmaf(h2f_hi(x.z), xb.y, t);
    t = __builtin_fmaf(h2f_lo(x.w), xb.z, t);
    t = __builtin_fmaf(h2f_hi(x.w), xb.w, t);
    acc = t;
    if (b == nb - 1 || last) {
      const float sum = wave_sum(acc);
      if (lane == 0) part[r * kWaves + wave] = sum;
      acc = 0.f;
    }
    if (++b == nb) {
      b = 0;
      ++r;
    }
  }
};

// one attention segment's consumer: even units are 4..8 keys of K, odd units
// the same keys of V; every key slot (lane group) keeps an online softmax
template <int G>
struct AttnConsume {
  float (&mrow)[G];
  float (&lrow)[G];
  float (&acc)[G][8];
  const float (&q)[G][8];
  float (&sc)[G];
  int ka, kc, kpl, kl, lpk, lane_active;
  KIE_DI void operator()(const uint4 x, int u, bool) {
    float v[8];
    v[0] = h2f_lo(x.x); v[1] = h2f_hi(x.x); v[2] = h2f_lo(x.y); v[3] = h2f_hi(x.y);
    v[4] = h2f_lo(x.z); v[5] = h2f_hi(x.z); v[6] = h2f_lo(x.w); v[7] = h2f_hi(x.w);
    if ((u & 1) == 0) {
      const int key = ka + (u >> 1) * kpl + kl;
      const bool ok = lane_active && key < kc;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float t = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) t = __builtin_fmaf(v[e], q[h][e], t);
        t = group_sum(t, lpk);
        sc[h] = ok ? t : -INFINITY;
      }
    } else {
#pragma unroll
      for (int h = 0; h < G; ++h) online_update(mrow[h], lrow[h], acc[h], sc[h], v);
    }
  }
};

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
template <int G>
__global__ void __launch_bounds__(kThreads, 1) kie_monokernel(const KParams P) {
  // Two separate LDS objects: the ring, written only by DMAs and read only by
  // ring_read(), and everything else.  Keeping them apart lets the compiler
  // prove that ordinary LDS accesses never alias an in-flight ring DMA.
  __shared__ float lds_main[kMainFloats];
  __shared__ Shared sh_static;
  __shared__ uint4 ring_lds[kWaves * kDepth * kWave];
  float* const lds_dyn = lds_main;
  const KParams& p = P;
  Dev D;
  D.p = &P;
  D.tid = threadIdx.x;
  D.wg = blockIdx.x;
  D.nwg = gridDim.x;
  D.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  D.lane = threadIdx.x & 63;
  D.sh = &sh_static;
  D.ring = ring_lds + D.wave * kDepth * kWave;
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
  int* wgrows = D.desc + kWaves * kWaveDesc;

  if (D.tid == 0) D.sh->abort = 0;
  // descriptors: every lane of a wave computes, lane 0 stores
  {
    int dsc[8], rows[2];
    const int kinds[5] = {PH_QKV, PH_O, PH_GU, PH_DOWN, PH_LM};
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      write_gemv_desc(p, kinds[k], D.nwg, D.wg, D.wave, dsc, rows);
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
  cur.s = 0;
  cur.ph = 0;
  cur.nph = 0;
  cur.done = 1;
  cur.rem = 0;
  cur.kind = PH_QKV;
  cur.st = 0; cur.kvh = 0; cur.ka = 0; cur.kc = 0; cur.nst = 0; cur.seg1 = 0; cur.l = 0;
  cur.b = 0; cur.nb = 1; cur.K8 = 0;
  cur.rowp = (const uint4*)p.W;
  cur.kb = p.kv;
  cur.vb = p.kv;
  int slot = 0;

  int token = 0;

  for (int s = 0; s < p.n_steps; ++s) {
    const uint32_t epoch = p.epoch0 + (uint32_t)s;
    const int pos = p.pos0 + s;
    // this step's attention descriptor (read by the consumer and the cursor)
    int* adesc = D.desc + D.wave * kWaveDesc + kConsumerAttn;
    {
      int ad[12];
      write_attn_desc(p, D.nwg, D.wg, D.wave, D.kpl, pos, ad);
#pragma unroll
      for (int i = 0; i < 12; ++i) adesc[i] = ad[i];
    }
    // restart the cursor on this step and fill the ring.  Every earlier ring
    // load has completed (the end-of-step polls waited for them), so the
    // slots can be reused in order from `slot`.
    __builtin_amdgcn_s_waitcnt(kWaitAllVm);
    cur.s = s;
    cur.ph = 0;
    cur.nph = nphases(p, s);
    cur.done = 0;
    cursor_enter(D, cur);
    for (int i = 0; i < kDepth; ++i) cursor_issue(D, cur, slot + i < kDepth ? slot + i : slot + i - kDepth);

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
      const uint16_t* e = p.W + p.pl.embed + (uint64_t)token * d;
      for (int i = D.tid; i < d; i += kThreads) xraw[i] = hbits2f(e[i]);
    }
    wg_sync();
    if (p.m.parallel) {
      const int r0 = wgrows[2 * 3], nr = wgrows[2 * 3 + 1];
      for (int t = D.tid; t < nr; t += kThreads) own[nr + t] = xraw[r0 + t];
      wg_sync();
    }

    if ((p.debug_flags & DBG_WAIT_NEVER) && D.wg == 0) {
      // wait on a word that no one writes: exercises the bounded wait
      if (D.tid == 0) {
        u64 dummy;
        spin_word(D, D.LMP + 2 * D.nwg - 1, 0xFFFFFFFFu, &dummy);
      }
      wg_sync();
      if (D.sh->abort) { __builtin_amdgcn_s_waitcnt(kWaitAllVm); return; }
    }

    const int nph = nphases(p, s);
    for (int ph = 0; ph < nph; ++ph) {
      const bool is_lm = ph == 5 * L;
      const int kind = is_lm ? PH_LM : phase_kind(p.m.parallel, ph % 5);
      const int l = is_lm ? L : ph / 5;
      const uint16_t* Wl = p.W + (uint64_t)(is_lm ? 0 : l) * p.pl.layer_stride;

      stamp(D, s, ph, 0);
      if (kind == PH_ATTN) {
        // ================= attention over the KV cache ==================
        float mrow[G], lrow[G], acc[G][8], q[G][8], sc[G];
        const int nseg = adesc[10];
        for (int sg = 0; sg < nseg; ++sg) {
          const int g = adesc[5 * sg + 0];
          const int ka = adesc[5 * sg + 1], kc = adesc[5 * sg + 2], nst = adesc[5 * sg + 3];
          const int has_pos = adesc[5 * sg + 4];
#pragma unroll
          for (int h = 0; h < G; ++h) {
            mrow[h] = -INFINITY;
            lrow[h] = 0.f;
            sc[h] = -INFINITY;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
          }
          // this lane's 8 query dims of every head in the group
          {
            const u64* qb = D.Q + (uint64_t)l * qd + (uint64_t)g * G * hd + D.dl * 8;
#pragma unroll
            for (int h = 0; h < G; ++h) {
              u64 qw[8];
              poll_words<8>(D, qb + h * hd, 1, 0xFFu, epoch, qw);
#pragma unroll
              for (int e = 0; e < 8; ++e) q[h][e] = ll_f(qw[e]);
            }
          }
          AttnConsume<G> ac{mrow, lrow, acc, q, sc, ka, kc, D.kpl, D.kl, D.lpk, D.lane_active};
          run_units(D, cur, slot, 2 * nst, ac);
          if (has_pos) {
            // current key and value (fp16-rounded) from the QKV epilogue
            const u64* kp = D.KC + (uint64_t)l * kvd + (uint64_t)g * hd + D.dl * 8;
            const u64* vp = D.VC + (uint64_t)l * kvd + (uint64_t)g * hd + D.dl * 8;
            u64 kw[8], vw[8];
            float kx[8], vx[8];
            poll_words<8>(D, kp, 1, 0xFFu, epoch, kw);
            poll_words<8>(D, vp, 1, 0xFFu, epoch, vw);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              kx[e] = ll_f(kw[e]);
              vx[e] = ll_f(vw[e]);
            }
            const bool mine = D.lane < D.lpk;
#pragma unroll
            for (int h = 0; h < G; ++h) {
              float t = 0.f;
#pragma unroll
              for (int e = 0; e < 8; ++e) t = __builtin_fmaf(kx[e], q[h][e], t);
              t = group_sum(t, D.lpk);
              if (mine) online_update(mrow[h], lrow[h], acc[h], t, vx);
            }
          }
          // merge this wave's key slots into lanes 0..lpk-1.  Only those
          // lanes accumulate; every other lane keeps its own slot's state, so
          // each slot is counted exactly once.
          const bool dst = D.lane < D.lpk;
          for (int k = 1; k < D.kpl; ++k) {
            const int src = D.lane + k * D.lpk;
#pragma unroll
            for (int h = 0; h < G; ++h) {
              const float mo = __shfl(mrow[h], src);
              const float lo = __shfl(lrow[h], src);
              float ao[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) ao[e] = __shfl(acc[h][e], src);
              if (dst) lse_merge(mrow[h], lrow[h], acc[h], mo, lo, ao);
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
        stamp(D, s, ph, 1);
        wg_sync();
        if (D.sh->abort) { __builtin_amdgcn_s_waitcnt(kWaitAllVm); return; }
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
        const int merge_g = adesc[11];
        if (merge_g >= 0) {
          const int g = merge_g;
          const int n_ctx = pos + 1;
          const int w_first = attn_owner(Hkv, n_ctx, D.nwg, g, 0);
          const int nrec = D.wg - w_first + 1;
          // 1. which records exist: mlw[r*4 + 3] = segment of record r or -1
          for (int r = D.tid; r < nrec; r += kThreads) {
            AttnSeg sgs[2];
            sgs[0] = AttnSeg{0, 0, 0};
            sgs[1] = AttnSeg{0, 0, 0};
            const int ns = attn_segments(Hkv, n_ctx, D.nwg, w_first + r, sgs);
            mlw[r * 4 + 3] = ns > 0 ? (float)((sgs[0].g == g) ? 0 : 1) : -1.f;
          }
          wg_sync();
          // 2. one poll round: every word of every record into LDS
          //    (record r, head h at recs[(r*G + h)*(hd+2) ...])
          float* recs = wrec;  // the wave records are consumed already
          const int rw = G * (hd + 2);
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
                const int si = (int)mlw[r * 4 + 3];
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
                if (*(volatile int*)&D.sh->abort) break;
                if (__hip_atomic_load(&D.state[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
                  D.sh->abort = 1;
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
          wg_sync();
          if (D.sh->abort) { __builtin_amdgcn_s_waitcnt(kWaitAllVm); return; }
          // 3. combine: o = sum_r exp2(m_r - M) O_r / sum_r exp2(m_r - M) l_r
          for (int t = D.tid; t < G * hd; t += kThreads) {
            const int h = t / hd, dd = t % hd;
            float M = -INFINITY;
            for (int r = 0; r < nrec; ++r) M = fmaxf(M, recs[(r * G + h) * (hd + 2)]);
            float Ls = 0.f, o = 0.f;
            for (int r = 0; r < nrec; ++r) {
              const float* rr = recs + (r * G + h) * (hd + 2);
              const float a = rr[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(rr[0] - M);
              Ls += a * rr[1];
              o += a * rr[2 + dd];
            }
            o = o / Ls;
            ll_storef(D.OB + (uint64_t)l * qd + (uint64_t)(g * G + h) * hd + dd, o, epoch);
          }
        }
        wg_sync();
        if (D.sh->abort) { __builtin_amdgcn_s_waitcnt(kWaitAllVm); return; }
        stamp(D, s, ph, 3);
        continue;
      }

      // ===================== GEMV phases =====================
      const int gi = gemv_index(kind);
      const int r0 = wgrows[2 * gi], nrows = wgrows[2 * gi + 1];
      // prologue: the input vector
      if (kind == PH_QKV) {
        if (p.m.parallel ? (l > p.m.delay) : (l > 0)) {
          const int xi = p.m.parallel ? l : 2 * l;
          poll_to_lds<false>(D, D.X + (uint64_t)xi * d, xraw, d, epoch);
          wg_sync();
          if (D.sh->abort) { __builtin_amdgcn_s_waitcnt(kWaitAllVm); return; }
        }
        rmsnorm_to_xs(D, xraw, Wl + p.pl.attn_norm, xs);
      } else if (kind == PH_GU) {
        if (!p.m.parallel) {
          poll_to_lds<false>(D, D.X + (uint64_t)(2 * l + 1) * d, xraw, d, epoch);
          wg_sync();
          if (D.sh->abort) { __builtin_amdgcn_s_waitcnt(kWaitAllVm); return; }
        }
        rmsnorm_to_xs(D, xraw, Wl + p.pl.mlp_norm, xs);
      } else if (kind == PH_O) {
        poll_to_lds<true>(D, D.OB + (uint64_t)l * qd, xs, qd, epoch);
        zero_tail(D, xs, qd);
      } else if (kind == PH_DOWN) {
        poll_to_lds<true>(D, D.HB + (uint64_t)l * F, xs, F, epoch);
        zero_tail(D, xs, F);
      } else {  // LM
        poll_to_lds<false>(D, D.X + (uint64_t)(2 * L) * d, xraw, d, epoch);
        wg_sync();
        if (D.sh->abort) { __builtin_amdgcn_s_waitcnt(kWaitAllVm); return; }
        rmsnorm_to_xs(D, xraw, p.W + p.pl.final_norm, xs);
      }
      for (int i = D.tid; i < nrows * kWaves; i += kThreads) part[i] = 0.f;
      wg_sync();
      if (D.sh->abort) { __builtin_amdgcn_s_waitcnt(kWaitAllVm); return; }
      stamp(D, s, ph, 1);

      {
        const int* gd = D.desc + D.wave * kWaveDesc + 8 * gi;
        GemvConsume c{(const float4*)xs, part, gd[6], gd[2], gd[4], D.lane, D.wave, 0.f};
        run_units(D, cur, slot, gd[3], c);
      }
      stamp(D, s, ph, 2);
      wg_sync();

      // epilogue
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
          const int rr = r0 + 2 * t;
          if (rr < qd + kvd) {
            const bool isq = rr < qd;
            const int base = isq ? 0 : qd;
            const int head = (rr - base) / hd;
            const int i = ((rr - base) % hd) >> 1;
            const float2 cs = rp[i];
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
          const float hval = y0 / (1.0f + expf(-y0)) * y1;
          ll_storef(D.HB + (uint64_t)l * F + (r0 >> 1) + t, hval, epoch);
        }
      } else if (kind == PH_O) {
        for (int t = D.tid; t < nrows; t += kThreads) {
          float y = 0.f;
#pragma unroll
          for (int w = 0; w < kWaves; ++w) y += part[t * kWaves + w];
          if (p.m.parallel) {
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
          if (p.m.parallel) {
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
          const int row = r0 + t;
          if (p.logits) p.logits[(uint64_t)out_step * V + row] = y;
          if (y > my_val || (y == my_val && row < my_idx)) {
            my_val = y;
            my_idx = row;
          }
        }
        for (int off = 32; off >= 1; off >>= 1) {
          const float ov = __shfl_xor(my_val, off);
          const int oi = __shfl_xor(my_idx, off);
          if (ov > my_val || (ov == my_val && oi < my_idx)) {
            my_val = ov;
            my_idx = oi;
          }
        }
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
          if (ov > bv || (ov == bv && oi < bi)) {
            bv = ov;
            bi = oi;
          }
        }
      }
      ll_storef(D.LMP + 2 * D.wg, bv, epoch);
      ll_store(D.LMP + 2 * D.wg + 1, (uint32_t)bi, epoch);
    }
    // every workgroup reads every partial and takes the same decision
    float* lv = xs;
    int* li = (int*)(xs + D.nwg);
    for (int t = D.tid; t < D.nwg; t += kThreads) {
      u64 ab[2];
      poll_words<2>(D, D.LMP + 2 * t, 1, 3u, epoch, ab);
      lv[t] = ll_f(ab[0]);
      li[t] = (int)(uint32_t)ab[1];
    }
    wg_sync();
    // every workgroup's release is now observed: one acquire (L1 and L2
    // invalidate) before this workgroup reads KV rows of the next step
    if (D.tid == 0) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      __builtin_amdgcn_s_waitcnt(kWaitAllVm);
    }
    wg_sync();
    if (D.sh->abort) { __builtin_amdgcn_s_waitcnt(kWaitAllVm); return; }
    stamp(D, s, tph, 1);
    if (lm) {
      if (D.tid == 0) {
        float bv = lv[0];
        int bi = li[0];
        for (int t = 1; t < D.nwg; ++t) {
          if (lv[t] > bv || (lv[t] == bv && li[t] < bi)) {
            bv = lv[t];
            bi = li[t];
          }
        }
        D.sh->token = bi;
      }
      wg_sync();
      token = D.sh->token;
      if (D.wg == 0 && D.tid == 0) {
        if (p.out) p.out[p.lm_mode == 1 ? 0 : s] = token;
        D.state[2] = token;
      }
    }
    wg_sync();
  }  // steps
  __builtin_amdgcn_s_waitcnt(kWaitAllVm);  // no ring DMA may outlive the workgroup
}

// fill with zeros (a graph-capturable replacement for a memset)
__global__ void kie_zero_kernel(uint4* p, uint64_t n16) {
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (uint64_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

}  // namespace kie

// ---------------------------------------------------------------------------
// host-side launch helpers (called by the C-ABI in kie_api.cpp)
// ---------------------------------------------------------------------------
static const void* kie_kernel_for(int G) {
  switch (G) {
    case 1: return (const void*)&kie::kie_monokernel<1>;
    case 2: return (const void*)&kie::kie_monokernel<2>;
    case 4: return (const void*)&kie::kie_monokernel<4>;
    default: return nullptr;
  }
}

extern "C" hipError_t kie_internal_launch(const kie::KParams* kp, int nwg, size_t lds_bytes, hipStream_t stream) {
  const void* fn = kie_kernel_for(kp->m.G);
  if (!fn) return hipErrorInvalidValue;
  (void)lds_bytes;  // all LDS is static
  void* args[] = {(void*)kp};
  return hipLaunchCooperativeKernel(fn, dim3(nwg), dim3(kie::kThreads), args, 0, stream);
}

extern "C" hipError_t kie_internal_zero(void* p, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  if (((uintptr_t)p & 15) || (bytes & 15)) return hipErrorInvalidValue;
  const uint64_t n16 = bytes / 16;
  const uint64_t want = (n16 + 255) / 256;
  const int blocks = (int)(want < 4096 ? want : 4096);
  hipLaunchKernelGGL(kie::kie_zero_kernel, dim3(blocks), dim3(256), 0, stream, (uint4*)p, n16);
  return hipGetLastError();
}

extern "C" hipError_t kie_internal_occupancy(int G, size_t lds_bytes, int* blocks_per_cu) {
  const void* fn = kie_kernel_for(G);
  if (!fn) return hipErrorInvalidValue;
  (void)lds_bytes;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, fn, kie::kThreads, 0);
}
