// Host side of the C ABI declared in include/kie.h: argument validation,
// buffer sizing, the weight packer, workspace set-up and the launches of the
// persistent decode kernel.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "kie.h"
#include "kie_layout.h"

// the decode kernel, built for each ring depth (kie_kernel.hip)
extern "C" hipError_t kie_internal_launch_ring8(const kie::KParams* kp, int nwg, size_t lds_bytes, hipStream_t stream);
extern "C" hipError_t kie_internal_launch_ring10(const kie::KParams* kp, int nwg, size_t lds_bytes, hipStream_t stream);
extern "C" hipError_t kie_internal_zero_ring8(void* p, size_t bytes, hipStream_t stream);
extern "C" hipError_t kie_internal_occupancy_ring8(int G, int parallel, size_t lds_bytes, int* blocks_per_cu);
extern "C" hipError_t kie_internal_occupancy_ring10(int G, int parallel, size_t lds_bytes, int* blocks_per_cu);
static_assert(kie::kRingBase == 8 && kie::kRingDeep == 10, "entry point names carry the ring depths");
extern "C" hipError_t kie_internal_prefill_chunk(const kie::PrefillArgs* a, hipStream_t stream);
extern "C" hipError_t kie_internal_noalloc_scratch(int device, void** ptr);

struct kie_ctx {
  kie_model_config cfg;
  kie::Dims m;
  int device = -1;
  int nwg = 256;
  kie::PackLayout pl;
  kie::WsLayout wl;
  int depth = kie::kRingBase;  // ring slots per wave of the kernel this context runs
  kie::LdsPlan lp;
  void* packed = nullptr;
  void* kv = nullptr;
  void* ws = nullptr;
  bool bound = false;
  bool loaded = false;
  int32_t pos = 0;
  uint32_t next_epoch = 1;  // epoch of the next decode step (0 = never written)
  uint64_t timeout_us = 2000000;
  uint32_t debug = 0;
  float temperature = 0.f;  // 0: greedy
  uint64_t seed = 0;
  int32_t launch_steps = 512;
  uint64_t* trace = nullptr;
  void* noalloc_scratch = nullptr;  // this device's kie_prefill_batched_noalloc scratch
  int32_t trace_steps = 0;
  double clock_khz = 100000.0;
  std::string err;
};

namespace {

constexpr int32_t kPrefillChunk = 2048;  // most prompt tokens per batched-prefill chunk

kie_status fail(kie_ctx* c, kie_status s, const std::string& msg) {
  if (c) c->err = msg;
  return s;
}

kie_status hip_fail(kie_ctx* c, hipError_t e, const char* what) {
  return fail(c, KIE_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

std::string check_config(const kie_model_config& c) {
  if (c.n_layers <= 0 || c.d_model <= 0 || c.n_heads <= 0 || c.n_kv_heads <= 0 || c.head_dim <= 0 ||
      c.ffn_dim <= 0 || c.vocab <= 0 || c.max_ctx <= 0)
    return "all sizes must be positive";
  if (c.n_heads % c.n_kv_heads) return "n_heads must be a multiple of n_kv_heads";
  if (c.head_dim % 8) return "head_dim must be a multiple of 8";
  if (c.d_model % 8 || (c.n_heads * c.head_dim) % 8 || c.ffn_dim % 8)
    return "d_model, n_heads*head_dim and ffn_dim must be multiples of 8";
  if (c.vocab % 2) return "vocab must be even (the LM head is stored as row pairs)";
  if (c.n_lanes <= 0 || c.n_heads % c.n_lanes || c.ffn_dim % c.n_lanes)
    return "n_lanes must divide n_heads and ffn_dim";
  if (c.parallel_block != 0 && c.parallel_block != 1) return "parallel_block must be 0 or 1";
  if (c.lane_delay < 0) return "lane_delay must be >= 0";
  if (!c.parallel_block && c.lane_delay) return "lane_delay needs parallel_block = 1";
  if (!(c.rms_eps >= 0.f) || !(c.rope_base > 1.0)) return "rms_eps must be >= 0 and rope_base > 1";
  return "";
}

kie::Dims make_dims(const kie_model_config& c) {
  kie::Dims m{};
  m.L = c.n_layers;
  m.d = c.d_model;
  m.H = c.n_heads;
  m.Hkv = c.n_kv_heads;
  m.hd = c.head_dim;
  m.F = c.ffn_dim;
  m.V = c.vocab;
  m.G = c.n_heads / c.n_kv_heads;
  m.max_ctx = c.max_ctx;
  m.parallel = c.parallel_block;
  m.delay = c.lane_delay;
  m.eps = c.rms_eps;
  return m;
}

// The phase order of a step (phase_at) against what each phase reads:
// every (kind, layer) once; QKV after the down projection that published its
// x; attention after its QKV; O after its attention; gate/up (sequential
// block) after O; down after its gate/up and its O.  Where the parallel block
// stages inputs in LDS (LdsPlan::hb) also: gate/up right after its QKV (the
// QKV prologue writes gate/up's input), O and down of a layer adjacent (the
// O prologue writes down's input, the O epilogue the rows down adds), and the
// QKV that an O prologue stages for after that O, with no other O between.
std::string check_phase_order(const kie::Dims& m, const kie::LdsPlan& lp) {
  const int L = m.L;
  std::vector<int> at(5 * (size_t)L, -1);  // (kind, layer) -> phase
  for (int ph = 0; ph < 5 * L; ++ph) {
    int k, l;
    kie::phase_at(lp.pipe, m.parallel, L, ph, &k, &l);
    if (k < 0 || k >= 5 || l < 0 || l >= L || at[5 * (size_t)l + k] >= 0) return "phase order repeats a phase";
    at[5 * (size_t)l + k] = ph;
  }
  auto P = [&](int k, int l) { return at[5 * (size_t)l + k]; };
  const bool staged = m.parallel && lp.hb >= 0 && m.G <= 2;
  for (int l = 0; l < L; ++l) {
    // the down projection that publishes the QKV input of layer l
    const int src = m.parallel ? (l > m.delay ? l - m.delay - 1 : -1) : l - 1;
    if (src >= 0 && P(kie::PH_DOWN, src) > P(kie::PH_QKV, l)) return "QKV before its input";
    if (P(kie::PH_ATTN, l) < P(kie::PH_QKV, l)) return "attention before its QKV";
    if (P(kie::PH_O, l) < P(kie::PH_ATTN, l)) return "O before its attention";
    if (!m.parallel && P(kie::PH_GU, l) < P(kie::PH_O, l)) return "gate/up before O";
    if (m.parallel && src >= 0 && P(kie::PH_DOWN, src) > P(kie::PH_GU, l)) return "gate/up before its input";
    if (P(kie::PH_DOWN, l) < P(kie::PH_GU, l) || P(kie::PH_DOWN, l) < P(kie::PH_O, l)) return "down before its inputs";
    if (!staged) continue;
    if (P(kie::PH_GU, l) != P(kie::PH_QKV, l) + 1) return "gate/up not right after its QKV";
    if (P(kie::PH_DOWN, l) != P(kie::PH_O, l) + 1) return "down not right after its O";
    const int ln = l + 1 + lp.pipe;  // the layer whose input the O prologue of layer l stages
    if (ln < L) {
      if (P(kie::PH_QKV, ln) < P(kie::PH_O, l)) return "staged QKV before the O that stages it";
      if (l + 1 < L && P(kie::PH_O, l + 1) < P(kie::PH_QKV, ln)) return "staged input overwritten before its QKV";
      const bool stage_x = m.delay > lp.pipe;  // as in the kernel: else the QKV polls x itself
      if (stage_x && ln > m.delay && P(kie::PH_DOWN, ln - m.delay - 1) > P(kie::PH_O, l))
        return "input staged before it is published";
    }
  }
  return "";
}

std::string check_supported(const kie::Dims& m, int nwg) {
  if (m.G != 1 && m.G != 2 && m.G != 4) return "query heads per KV head must be 1, 2 or 4";
  if (m.hd / 8 > 64) return "head_dim above 512 is not supported";
  if (m.d > kie::kGainRegs * kie::kThreads) return "d_model above 4096 is not supported";
  if (m.Hkv > nwg) return "more KV heads than workgroups";
  const int budget = kie::main_floats(kie::ring_depth_for(m, nwg));
  const kie::LdsPlan lp = kie::lds_plan(m, nwg, budget);
  if (lp.total_floats > budget) return "model needs more LDS than the kernel reserves";
  const std::string po = check_phase_order(m, lp);
  if (!po.empty()) return po;
  const uint64_t lim = 0x7FFFFFFFull;
  if ((uint64_t)m.Hkv * (uint64_t)(m.max_ctx + 1) * (uint64_t)nwg > lim) return "KV heads x context too large";
  if ((uint64_t)m.V * (uint64_t)nwg > lim || (uint64_t)2 * m.F * (uint64_t)nwg > lim)
    return "vocab or ffn too large for the partition arithmetic";
  if ((uint64_t)m.V * (uint64_t)m.d >= (1ull << 32)) return "LM head too large";
  return "";
}

// ---------------------------------------------------------------------------
// packer
// ---------------------------------------------------------------------------
void copy_rows(uint16_t* dst, const uint16_t* src, size_t n) { std::memcpy(dst, src, n * sizeof(uint16_t)); }

// n rows of k columns into the row-pair chunk layout (kie_layout.h), packed
// row r read from src_row(r); dst is zeroed beforehand, so the columns past
// k stay zero
template <class RowFn>
void pack_matrix(uint16_t* dst, size_t n, int k, RowFn src_row) {
  const int nb = kie::col_blocks(k);
  for (size_t r = 0; r < n; ++r) {
    const uint16_t* s = src_row(r);
    for (int b = 0; b < nb; ++b) {
      const int c0 = b * kie::kPairCols;
      copy_rows(dst + kie::packed_at(r, c0, k), s + c0, (size_t)std::min(kie::kPairCols, k - c0));
    }
  }
}

bool weights_complete(const kie_model_config& c, const kie_weights* w) {
  if (!w || !w->embed || !w->lm_head || !w->final_norm || !w->attn_norm || !w->wq || !w->wk || !w->wv || !w->wo ||
      !w->mlp_norm || !w->w_gate || !w->w_up || !w->w_down)
    return false;
  for (int l = 0; l < c.n_layers; ++l)
    if (!w->attn_norm[l] || !w->wq[l] || !w->wk[l] || !w->wv[l] || !w->wo[l] || !w->mlp_norm[l] || !w->w_gate[l] ||
        !w->w_up[l] || !w->w_down[l])
      return false;
  return true;
}

// pack layer l into dst (layer_stride elements)
void pack_layer(const kie::Dims& m, const kie::PackLayout& pl, const kie_weights* w, int l, uint16_t* dst) {
  const size_t d = m.d, qd = (size_t)m.H * m.hd, F = m.F;
  std::memset(dst, 0, pl.layer_stride * sizeof(uint16_t));
  copy_rows(dst + pl.attn_norm, w->attn_norm[l], d);
  const size_t rows = (size_t)(m.H + 2 * m.Hkv) * m.hd;
  pack_matrix(dst + pl.wqkv, rows, m.d, [&](size_t r) {
    int which, src;
    kie::qkv_source_row(m, (int)r, &which, &src);
    const uint16_t* s = which == 0 ? w->wq[l] : which == 1 ? w->wk[l] : w->wv[l];
    return s + (size_t)src * d;
  });
  pack_matrix(dst + pl.wo, d, (int)qd, [&](size_t r) { return w->wo[l] + r * qd; });
  copy_rows(dst + pl.mlp_norm, w->mlp_norm[l], d);
  pack_matrix(dst + pl.wgu, 2 * F, m.d,
              [&](size_t r) { return (r & 1 ? w->w_up[l] : w->w_gate[l]) + (r >> 1) * d; });
  pack_matrix(dst + pl.wd, d, (int)F, [&](size_t r) { return w->w_down[l] + r * F; });
}

// the part after the layers: final_norm, lm_head, embed
void pack_tail(const kie::Dims& m, const kie::PackLayout& pl, const kie_weights* w, uint16_t* dst_at_final_norm) {
  const uint64_t base = pl.final_norm;
  std::memset(dst_at_final_norm, 0, (pl.total - base) * sizeof(uint16_t));
  copy_rows(dst_at_final_norm + (pl.final_norm - base), w->final_norm, m.d);
  pack_matrix(dst_at_final_norm + (pl.lm_head - base), (size_t)m.V, m.d,
              [&](size_t r) { return w->lm_head + r * (size_t)m.d; });
  copy_rows(dst_at_final_norm + (pl.embed - base), w->embed, (size_t)m.V * m.d);
}

// RoPE table: (cos, sin) of pos * base^(-2i/hd), computed in double
void rope_table(const kie::Dims& m, double base, std::vector<float>& out) {
  const int half = m.hd / 2;
  out.resize((size_t)m.max_ctx * half * 2);
  std::vector<double> inv(half);
  for (int i = 0; i < half; ++i) inv[i] = std::pow(base, -2.0 * i / m.hd);
  for (int p = 0; p < m.max_ctx; ++p)
    for (int i = 0; i < half; ++i) {
      const double a = (double)p * inv[i];
      out[((size_t)p * half + i) * 2] = (float)std::cos(a);
      out[((size_t)p * half + i) * 2 + 1] = (float)std::sin(a);
    }
}

kie::KParams base_params(const kie_ctx* c) {
  kie::KParams kp{};
  kp.m = c->m;
  kp.pl = c->pl;
  kp.wl = c->wl;
  kp.lp = c->lp;
  kp.W = (const uint16_t*)c->packed;
  kp.kv = (uint16_t*)c->kv;
  kp.ws = (uint8_t*)c->ws;
  kp.timeout_ticks = (uint64_t)((double)c->timeout_us * c->clock_khz / 1000.0);
  if (kp.timeout_ticks == 0) kp.timeout_ticks = 1;
  kp.debug_flags = c->debug;
  kp.trace = c->trace;
  kp.trace_steps = c->trace_steps;
  kp.sample = c->temperature > 0.f ? 1 : 0;
  kp.inv_temp = c->temperature > 0.f ? 1.0f / c->temperature : 1.0f;
  kp.seed_lo = (uint32_t)c->seed;
  kp.seed_hi = (uint32_t)(c->seed >> 32);
  return kp;
}

kie_status ready(kie_ctx* c) {
  if (!c) return KIE_ERR_INVALID_ARG;
  if (c->device < 0) return fail(c, KIE_ERR_STATE, "host-only context");
  if (!c->bound) return fail(c, KIE_ERR_STATE, "memory not bound");
  if (!c->loaded) return fail(c, KIE_ERR_STATE, "weights not loaded");
  return KIE_OK;
}

kie_status launch(kie_ctx* c, kie::KParams& kp, hipStream_t st) {
  hipError_t e = hipSetDevice(c->device);
  if (e != hipSuccess) return hip_fail(c, e, "hipSetDevice");
  e = c->depth == kie::kRingDeep ? kie_internal_launch_ring10(&kp, c->nwg, 0, st)
                                 : kie_internal_launch_ring8(&kp, c->nwg, 0, st);
  if (e != hipSuccess) return hip_fail(c, e, "monokernel launch");
  c->next_epoch += (uint32_t)kp.n_steps;
  return KIE_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
extern "C" {

kie_status kie_create(const kie_model_config* cfg, int device, kie_ctx** out) {
  if (!cfg || !out) return KIE_ERR_INVALID_ARG;
  *out = nullptr;
  const std::string msg = check_config(*cfg);
  if (!msg.empty()) {
    std::fprintf(stderr, "kie_create: %s\n", msg.c_str());
    return KIE_ERR_INVALID_ARG;
  }
  kie_ctx* c = new kie_ctx();
  c->cfg = *cfg;
  c->m = make_dims(*cfg);
  c->device = device;
  if (device >= 0) {
    hipError_t e = hipSetDevice(device);
    hipDeviceProp_t prop;
    if (e == hipSuccess) e = hipGetDeviceProperties(&prop, device);
    if (e != hipSuccess) {
      std::fprintf(stderr, "kie_create: %s\n", hipGetErrorString(e));
      delete c;
      return KIE_ERR_HIP;
    }
    c->nwg = prop.multiProcessorCount;
    int khz = 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, device) == hipSuccess && khz > 0)
      c->clock_khz = khz;
  }
  const std::string sup = check_supported(c->m, c->nwg);
  if (!sup.empty()) {
    std::fprintf(stderr, "kie_create: %s\n", sup.c_str());
    delete c;
    return KIE_ERR_UNSUPPORTED;
  }
  if (device >= 0) {
    int per_cu = 0;
    const int depth = kie::ring_depth_for(c->m, c->nwg);
    hipError_t e = depth == kie::kRingDeep ? kie_internal_occupancy_ring10(c->m.G, c->m.parallel, 0, &per_cu)
                                           : kie_internal_occupancy_ring8(c->m.G, c->m.parallel, 0, &per_cu);
    if (e != hipSuccess || per_cu < 1) {
      std::fprintf(stderr, "kie_create: kernel does not fit a compute unit (%s)\n",
                   e == hipSuccess ? "occupancy 0" : hipGetErrorString(e));
      delete c;
      return KIE_ERR_UNSUPPORTED;
    }
  }
  if (device >= 0) {
    // the device address of this GPU's no-allocation scratch (the device is
    // current: hipSetDevice above)
    const hipError_t e = kie_internal_noalloc_scratch(device, &c->noalloc_scratch);
    if (e != hipSuccess) {
      std::fprintf(stderr, "kie_create: no-allocation scratch: %s\n", hipGetErrorString(e));
      delete c;
      return KIE_ERR_HIP;
    }
  }
  c->pl = kie::pack_layout(c->m);
  c->wl = kie::ws_layout(c->m, c->nwg);
  c->depth = kie::ring_depth_for(c->m, c->nwg);
  c->lp = kie::lds_plan(c->m, c->nwg, kie::main_floats(c->depth));
  *out = c;
  return KIE_OK;
}

kie_status kie_query_sizes(const kie_ctx* c, size_t* packed, size_t* kv, size_t* ws) {
  if (!c) return KIE_ERR_INVALID_ARG;
  if (packed) *packed = (size_t)c->pl.total * 2;
  if (kv) *kv = (size_t)kie::kv_alloc_elems(c->m) * 2;
  if (ws) *ws = (size_t)c->wl.total;
  return KIE_OK;
}

kie_status kie_bind_memory(kie_ctx* c, void* d_packed, void* d_kv, void* d_ws) {
  if (!c) return KIE_ERR_INVALID_ARG;
  if (c->device < 0) return fail(c, KIE_ERR_STATE, "host-only context");
  if (!d_packed || !d_kv || !d_ws) return fail(c, KIE_ERR_INVALID_ARG, "null device pointer");
  if (((uintptr_t)d_packed | (uintptr_t)d_kv | (uintptr_t)d_ws) & 255)
    return fail(c, KIE_ERR_INVALID_ARG, "device buffers must be 256-byte aligned");
  hipError_t e = hipSetDevice(c->device);
  if (e != hipSuccess) return hip_fail(c, e, "hipSetDevice");
  c->packed = d_packed;
  c->kv = d_kv;
  c->ws = d_ws;
  c->bound = true;
  c->loaded = false;
  c->pos = 0;
  c->next_epoch = 1;
  // clear state and exchange words, upload the RoPE table
  uint8_t* w = (uint8_t*)d_ws;
  if ((e = kie_internal_zero_ring8(w + c->wl.state, 256, nullptr)) != hipSuccess) return hip_fail(c, e, "clear state");
  if ((e = kie_internal_zero_ring8(w + c->wl.ll_begin, c->wl.ll_end - c->wl.ll_begin, nullptr)) != hipSuccess)
    return hip_fail(c, e, "clear exchange words");
  std::vector<float> rope;
  rope_table(c->m, c->cfg.rope_base, rope);
  if ((e = hipMemcpy(w + c->wl.rope, rope.data(), rope.size() * sizeof(float), hipMemcpyHostToDevice)) != hipSuccess)
    return hip_fail(c, e, "upload RoPE table");
  if ((e = hipDeviceSynchronize()) != hipSuccess) return hip_fail(c, e, "bind");
  return KIE_OK;
}

kie_status kie_load_weights(kie_ctx* c, const kie_weights* src, void* stream) {
  if (!c) return KIE_ERR_INVALID_ARG;
  if (c->device < 0) return fail(c, KIE_ERR_STATE, "host-only context");
  if (!c->bound) return fail(c, KIE_ERR_STATE, "memory not bound");
  if (!weights_complete(c->cfg, src)) return fail(c, KIE_ERR_INVALID_ARG, "missing weight pointer");
  hipError_t e = hipSetDevice(c->device);
  if (e != hipSuccess) return hip_fail(c, e, "hipSetDevice");
  hipStream_t st = (hipStream_t)stream;
  if ((e = hipStreamSynchronize(st)) != hipSuccess) return hip_fail(c, e, "stream sync");
  std::vector<uint16_t> buf(c->pl.layer_stride);
  uint16_t* dst = (uint16_t*)c->packed;
  for (int l = 0; l < c->m.L; ++l) {
    pack_layer(c->m, c->pl, src, l, buf.data());
    e = hipMemcpy(dst + (size_t)l * c->pl.layer_stride, buf.data(), buf.size() * 2, hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(c, e, "upload layer");
  }
  std::vector<uint16_t> tail(c->pl.total - c->pl.final_norm);
  pack_tail(c->m, c->pl, src, tail.data());
  e = hipMemcpy(dst + c->pl.final_norm, tail.data(), tail.size() * 2, hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(c, e, "upload head");
  c->loaded = true;
  return KIE_OK;
}

kie_status kie_prefill(kie_ctx* c, const int32_t* d_prompt, int32_t n, int32_t* d_next, float* d_logits,
                       void* stream) {
  kie_status s = ready(c);
  if (s != KIE_OK) return s;
  if (!d_prompt || n <= 0) return fail(c, KIE_ERR_INVALID_ARG, "empty prompt");
  if ((int64_t)c->pos + n > c->m.max_ctx) return fail(c, KIE_ERR_CAPACITY, "prompt exceeds max_ctx");
  hipStream_t st = (hipStream_t)stream;
  for (int32_t off = 0; off < n;) {
    const int32_t chunk = std::min<int32_t>(c->launch_steps, n - off);
    const bool last = off + chunk == n;
    kie::KParams kp = base_params(c);
    kp.forced = d_prompt + off;
    kp.out = last ? d_next : nullptr;
    kp.logits = last ? d_logits : nullptr;
    kp.n_steps = chunk;
    kp.pos0 = c->pos;
    kp.lm_mode = last ? 1 : 2;
    kp.first_from_state = 0;
    kp.epoch0 = c->next_epoch;
    if ((s = launch(c, kp, st)) != KIE_OK) return s;
    c->pos += chunk;
    off += chunk;
  }
  return KIE_OK;
}

kie_status kie_prefill_scratch_bytes(const kie_ctx* c, int32_t chunk_tokens, size_t* bytes) {
  if (!c || !bytes || chunk_tokens <= 0) return KIE_ERR_INVALID_ARG;
  *bytes = (size_t)chunk_tokens * kie::pf_floats_per_token(c->m) * sizeof(float);
  return KIE_OK;
}

namespace {
kie_status prefill_batched(kie_ctx* c, const int32_t* d_prompt, int32_t n, int32_t* d_next, float* d_logits,
                           void* d_scratch, size_t scratch_bytes, void* stream) {
  kie_status s = ready(c);
  if (s != KIE_OK) return s;
  if (!d_prompt || n <= 0) return fail(c, KIE_ERR_INVALID_ARG, "empty prompt");
  if ((int64_t)c->pos + n > c->m.max_ctx) return fail(c, KIE_ERR_CAPACITY, "prompt exceeds max_ctx");
  // shapes the batched kernels do not take run token by token; so does a
  // one-token prompt
  const bool batched = n > 1 && c->m.hd <= 512 && (c->m.hd % 8) == 0 && (c->m.F % 4) == 0;
  if (!batched) return kie_prefill(c, d_prompt, n, d_next, d_logits, stream);
  if (!d_scratch || ((uintptr_t)d_scratch & 15))
    return fail(c, KIE_ERR_INVALID_ARG, "prefill scratch must be a 16-byte aligned device buffer");
  const uint64_t per_token = kie::pf_floats_per_token(c->m) * sizeof(float);
  const int64_t fit = (int64_t)(scratch_bytes / per_token);
  if (fit < 1) return fail(c, KIE_ERR_INVALID_ARG, "prefill scratch holds less than one token (kie_prefill_scratch_bytes)");
  const int32_t cmax = (int32_t)std::min<int64_t>(fit, kPrefillChunk);
  hipStream_t st = (hipStream_t)stream;
  kie::PrefillArgs a{};
  a.m = c->m;
  a.pl = c->pl;
  a.W = (const uint16_t*)c->packed;
  a.kv = (uint16_t*)c->kv;
  a.rope = (const float2*)((uint8_t*)c->ws + c->wl.rope);
  a.state = (int32_t*)((uint8_t*)c->ws + c->wl.state);
  a.scratch = (float*)d_scratch;
  for (int32_t off = 0; off < n - 1;) {
    const int32_t C = std::min<int32_t>(cmax, n - 1 - off);
    a.tokens = d_prompt + off;
    a.C = C;
    a.pos0 = c->pos + off;
    const hipError_t e = kie_internal_prefill_chunk(&a, st);
    if (e != hipSuccess) return hip_fail(c, e, "batched prefill launch");
    off += C;
  }
  c->pos += n - 1;
  // the last prompt token goes through the decode kernel: LM head, the
  // greedy or sampled t1, its logits, and the pending-token state
  return kie_prefill(c, d_prompt + n - 1, 1, d_next, d_logits, stream);
}
}  // namespace

kie_status kie_prefill_batched(kie_ctx* c, const int32_t* d_prompt, int32_t n, int32_t* d_next, float* d_logits,
                               void* d_scratch, size_t scratch_bytes, void* stream) {
  return prefill_batched(c, d_prompt, n, d_next, d_logits, d_scratch, scratch_bytes, stream);
}

kie_status kie_prefill_batched_noalloc(kie_ctx* c, const int32_t* d_prompt, int32_t n, int32_t* d_next,
                                       float* d_logits, void* stream) {
  kie_status s = ready(c);
  if (s != KIE_OK) return s;
  if (!c->noalloc_scratch) return fail(c, KIE_ERR_STATE, "no-allocation scratch not available on this device");
  const uint64_t per_token = kie::pf_floats_per_token(c->m) * sizeof(float);
  if (per_token > kie::kNoAllocScratchBytes)
    return fail(c, KIE_ERR_UNSUPPORTED,
                "one prompt token needs " + std::to_string(per_token) + " bytes of prefill scratch, more than the " +
                    std::to_string(kie::kNoAllocScratchBytes) + " bytes of the no-allocation scratch");
  return prefill_batched(c, d_prompt, n, d_next, d_logits, c->noalloc_scratch, kie::kNoAllocScratchBytes, stream);
}

kie_status kie_decode(kie_ctx* c, int32_t n, int32_t* d_out, const int32_t* d_forced, float* d_logits,
                      void* stream) {
  kie_status s = ready(c);
  if (s != KIE_OK) return s;
  if (n <= 0) return fail(c, KIE_ERR_INVALID_ARG, "n_tokens must be >= 1");
  if ((int64_t)c->pos + n > c->m.max_ctx) return fail(c, KIE_ERR_CAPACITY, "decode exceeds max_ctx");
  hipStream_t st = (hipStream_t)stream;
  for (int32_t off = 0; off < n;) {
    const int32_t chunk = std::min<int32_t>(c->launch_steps, n - off);
    kie::KParams kp = base_params(c);
    kp.forced = d_forced ? d_forced + off : nullptr;
    kp.out = d_out ? d_out + off : nullptr;
    kp.logits = d_logits ? d_logits + (size_t)off * c->m.V : nullptr;
    kp.n_steps = chunk;
    kp.pos0 = c->pos;
    kp.lm_mode = 0;
    kp.first_from_state = 1;
    kp.epoch0 = c->next_epoch;
    if ((s = launch(c, kp, st)) != KIE_OK) return s;
    c->pos += chunk;
    off += chunk;
  }
  return KIE_OK;
}

kie_status kie_set_position(kie_ctx* c, int32_t pos, int32_t next_token, void* stream) {
  if (!c) return KIE_ERR_INVALID_ARG;
  if (pos < 0 || pos > c->m.max_ctx) return fail(c, KIE_ERR_INVALID_ARG, "position out of range");
  if (next_token < 0 || next_token >= c->m.V) return fail(c, KIE_ERR_INVALID_ARG, "token out of range");
  if (c->device < 0 || !c->bound) return fail(c, KIE_ERR_STATE, "memory not bound");
  hipError_t e = hipSetDevice(c->device);
  if (e == hipSuccess)
    e = hipMemsetD32Async((hipDeviceptr_t)((uint8_t*)c->ws + c->wl.state + 8), next_token, 1, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(c, e, "set token");
  c->pos = pos;
  return KIE_OK;
}

kie_status kie_sync_status(kie_ctx* c, void* stream) {
  if (!c) return KIE_ERR_INVALID_ARG;
  if (c->device < 0 || !c->bound) return fail(c, KIE_ERR_STATE, "memory not bound");
  hipError_t e = hipSetDevice(c->device);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(c, e, "stream sync");
  int32_t st[2] = {0, 0};
  e = hipMemcpy(st, (uint8_t*)c->ws + c->wl.state, sizeof(st), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(c, e, "read status");
  if (st[0] == 0 && st[1] == 0) return KIE_OK;
  const int32_t zero[2] = {0, 0};
  e = hipMemcpy((uint8_t*)c->ws + c->wl.state, zero, sizeof(zero), hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(c, e, "clear status");
  // an aborted launch leaves exchange words and arrival counters part-way
  // through a step: start the exchange state over (the KV cache is kept)
  e = kie_internal_zero_ring8((uint8_t*)c->ws + c->wl.ll_begin, c->wl.ll_end - c->wl.ll_begin, nullptr);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(c, e, "reset exchange state");
  c->next_epoch = 1;
  if (st[0] == kie::DEV_BAD_TOKEN) return fail(c, KIE_ERR_BAD_TOKEN, "a token id outside [0, vocab) reached the kernel");
  if (st[0] == kie::DEV_RANGE)
    return fail(c, KIE_ERR_RANGE, "a prefill activation outside the fp16 range (|a| > 65504 or not finite)");
  return fail(c, KIE_ERR_TIMEOUT, "a wait inside the decode kernel timed out");
}

kie_status kie_set_timeout_us(kie_ctx* c, uint64_t us) {
  if (!c || us == 0) return KIE_ERR_INVALID_ARG;
  c->timeout_us = us;
  return KIE_OK;
}

kie_status kie_set_sampling(kie_ctx* c, float temperature, uint64_t seed) {
  if (!c) return KIE_ERR_INVALID_ARG;
  if (!std::isfinite(temperature) || temperature < 0.f)
    return fail(c, KIE_ERR_INVALID_ARG, "temperature must be finite and >= 0 (0 = greedy)");
  c->temperature = temperature;
  c->seed = seed;
  return KIE_OK;
}

kie_status kie_set_debug_flags(kie_ctx* c, uint32_t flags) {
  if (!c) return KIE_ERR_INVALID_ARG;
  c->debug = flags;
  return KIE_OK;
}

kie_status kie_set_trace(kie_ctx* c, void* d_trace, int32_t steps) {
  if (!c || steps < 0 || (steps > 0 && !d_trace)) return KIE_ERR_INVALID_ARG;
  c->trace = (uint64_t*)d_trace;
  c->trace_steps = d_trace ? steps : 0;
  return KIE_OK;
}

kie_status kie_phase_order(const kie_model_config* cfg, int32_t nwg, int32_t* kind, int32_t* layer, int32_t n) {
  if (!cfg || nwg <= 0 || !kind || !layer || !check_config(*cfg).empty()) return KIE_ERR_INVALID_ARG;
  const kie::Dims m = make_dims(*cfg);
  if (n < 5 * m.L + 1) return KIE_ERR_INVALID_ARG;
  if (!check_supported(m, nwg).empty()) return KIE_ERR_UNSUPPORTED;
  const kie::LdsPlan lp = kie::lds_plan(m, nwg, kie::main_floats(kie::ring_depth_for(m, nwg)));
  for (int ph = 0; ph < 5 * m.L; ++ph) {
    int k, l;
    kie::phase_at(lp.pipe, m.parallel, m.L, ph, &k, &l);
    kind[ph] = k;
    layer[ph] = l;
  }
  kind[5 * m.L] = kie::PH_LM;
  layer[5 * m.L] = m.L;
  return KIE_OK;
}

// packed row r of the fused QKV matrix (all q rows, then all k rows, then
// all v rows; qkv_source_row) -> which = 0 q, 1 k, 2 v and head (the query
// head for q, the KV head for k and v)
static void qkv_row_head(const kie::Dims& m, int r, int* which, int* head) {
  const int qd = m.H * m.hd, kvd = m.Hkv * m.hd;
  *which = r < qd ? 0 : r < qd + kvd ? 1 : 2;
  *head = (r - (*which == 0 ? 0 : *which == 1 ? qd : qd + kvd)) / m.hd;
}

kie_status kie_lane_placement(const kie_model_config* cfg, int32_t nwg, int32_t* lane_lo, int32_t* lane_hi) {
  if (!cfg || nwg <= 0 || !lane_lo || !lane_hi || !check_config(*cfg).empty()) return KIE_ERR_INVALID_ARG;
  const kie::Dims m = make_dims(*cfg);
  if (!check_supported(m, nwg).empty()) return KIE_ERR_UNSUPPORTED;
  const int qpl = m.H / cfg->n_lanes, fpl = m.F / cfg->n_lanes;  // query heads, FFN columns per lane
  for (int w = 0; w < nwg; ++w) {
    int lo[3] = {-1, -1, -1}, hi[3] = {-1, -1, -1};
    // lanes of the query heads [h0, h1] (kind k)
    auto take = [&](int k, int h0, int h1) {
      lo[k] = lo[k] < 0 ? h0 / qpl : std::min(lo[k], h0 / qpl);
      hi[k] = std::max(hi[k], h1 / qpl);
    };
    int r0, r1;
    kie::gemv_rows_any(m, kie::PH_QKV, nwg, w, &r0, &r1);
    for (int r = r0; r < r1; ++r) {
      int which, head;
      qkv_row_head(m, r, &which, &head);
      if (which == 0) take(0, head, head);
      else take(0, head * m.G, head * m.G + m.G - 1);
    }
    const int g = kie::attn_head(m.Hkv, nwg, w);  // the workgroup's KV head (attention group)
    take(1, g * m.G, g * m.G + m.G - 1);
    kie::gemv_rows_any(m, kie::PH_GU, nwg, w, &r0, &r1);
    if (r1 > r0) {  // packed gate/up row pair f is FFN column f
      lo[2] = (r0 / 2) / fpl;
      hi[2] = ((r1 - 1) / 2) / fpl;
    }
    for (int k = 0; k < 3; ++k) {
      lane_lo[k * nwg + w] = lo[k];
      lane_hi[k * nwg + w] = hi[k];
    }
  }
  return KIE_OK;
}

kie_status kie_ring_depth(const kie_model_config* cfg, int32_t nwg, int32_t* depth) {
  if (!cfg || nwg <= 0 || !depth || !check_config(*cfg).empty()) return KIE_ERR_INVALID_ARG;
  const kie::Dims m = make_dims(*cfg);
  if (!check_supported(m, nwg).empty()) return KIE_ERR_UNSUPPORTED;
  *depth = kie::ring_depth_for(m, nwg);
  return KIE_OK;
}

kie_status kie_set_launch_steps(kie_ctx* c, int32_t steps) {
  if (!c || steps <= 0) return KIE_ERR_INVALID_ARG;
  c->launch_steps = steps;
  return KIE_OK;
}

kie_status kie_pack_weights_host(const kie_model_config* cfg, const kie_weights* src, void* host_dst) {
  if (!cfg || !host_dst) return KIE_ERR_INVALID_ARG;
  if (!check_config(*cfg).empty()) return KIE_ERR_INVALID_ARG;
  if (!weights_complete(*cfg, src)) return KIE_ERR_INVALID_ARG;
  const kie::Dims m = make_dims(*cfg);
  const kie::PackLayout pl = kie::pack_layout(m);
  uint16_t* dst = (uint16_t*)host_dst;
  for (int l = 0; l < m.L; ++l) pack_layer(m, pl, src, l, dst + (size_t)l * pl.layer_stride);
  pack_tail(m, pl, src, dst + pl.final_norm);
  return KIE_OK;
}

kie_status kie_launch_info(const kie_ctx* c, int32_t* nwg, int32_t* threads, int32_t* lds, int64_t* qkv_off,
                           int64_t* lm_off) {
  if (!c) return KIE_ERR_INVALID_ARG;
  if (nwg) *nwg = c->nwg;
  if (threads) *threads = kie::kThreads;
  if (lds) *lds = kie::main_floats(c->depth) * 4 + kie::kWaves * c->depth * 1024;
  if (qkv_off) *qkv_off = (int64_t)c->pl.wqkv;
  if (lm_off) *lm_off = (int64_t)c->pl.lm_head;
  return KIE_OK;
}

kie_status kie_validate_schedule(const kie_model_config* cfg, int32_t nwg, int32_t n_ctx, char* msg, size_t msg_len) {
  auto bad = [&](const std::string& s) {
    if (msg && msg_len) std::snprintf(msg, msg_len, "%s", s.c_str());
    return KIE_ERR_INVALID_ARG;
  };
  if (!cfg || nwg <= 0 || n_ctx <= 0) return bad("bad arguments");
  const std::string cm = check_config(*cfg);
  if (!cm.empty()) return bad(cm);
  const kie::Dims m = make_dims(*cfg);
  const std::string sup = check_supported(m, nwg);
  if (!sup.empty()) return bad(sup);
  // GEMV: rows and (row, block) units
  const int kinds[5] = {kie::PH_QKV, kie::PH_O, kie::PH_GU, kie::PH_DOWN, kie::PH_LM};
  for (int k : kinds) {
    const kie::GemvShape sh = kie::gemv_shape(m, k);
    std::vector<int> owner(sh.rows, -1);
    for (int w = 0; w < nwg; ++w) {
      int r0, r1;
      kie::gemv_rows_any(m, k, nwg, w, &r0, &r1);
      if (r0 % sh.unit_rows || r1 % sh.unit_rows) return bad("row range splits a row group");
      for (int r = r0; r < r1; ++r) {
        if (r < 0 || r >= sh.rows || owner[r] != -1) return bad("GEMV row owned twice or out of range");
        owner[r] = w;
      }
      // chunks of the workgroup's packed stretch: contiguous per wave, every
      // packed element of its row pairs read by exactly one wave
      const int nch = kie::gemv_chunks(r1 - r0, sh.K);
      if ((uint64_t)nch * kie::kBlock != kie::packed_elems((uint64_t)(r1 - r0), sh.K))
        return bad("chunk count does not match the workgroup rows");
      if (kie::packed_at((uint64_t)r0, 0, sh.K) + (uint64_t)nch * kie::kBlock !=
          kie::packed_at((uint64_t)r1, 0, sh.K))
        return bad("workgroup chunks are not contiguous");
      int prev_end = 0;
      for (int wave = 0; wave < kie::kWaves; ++wave) {
        int c0, c1;
        kie::gemv_wave_chunks(r1 - r0, sh.K, wave, &c0, &c1);
        if (c0 != prev_end || c1 < c0) return bad("wave chunk ranges not contiguous");
        prev_end = c1;
      }
      if (prev_end != nch) return bad("wave chunks do not cover the workgroup rows");
    }
    for (int r = 0; r < sh.rows; ++r)
      if (owner[r] < 0) return bad("GEMV row not owned");
  }
  // attention: keys, segments, mergers
  const int kpl = kie::attn_kpl(m.hd);
  std::vector<int> key_owner((size_t)m.Hkv * n_ctx, 0);
  std::vector<int> mergers(m.Hkv, 0);
  const int pos = n_ctx - 1;
  for (int w = 0; w < nwg; ++w) {
    kie::AttnSeg seg[2];
    const int ns = kie::attn_segments(m.Hkv, n_ctx, nwg, w, seg);
    if (ns > 1) return bad("a workgroup meets more than one KV head");
    for (int s = 0; s < ns; ++s) {
      if (seg[s].g != kie::attn_head(m.Hkv, nwg, w)) return bad("segment outside the workgroup's head");
      if (seg[s].tb == n_ctx) mergers[seg[s].g]++;
      for (int wave = 0; wave < kie::kWaves; ++wave) {
        int wa, wb;
        kie::wave_split(seg[s].tb - seg[s].ta, wave, &wa, &wb);
        wa += seg[s].ta;
        wb += seg[s].ta;
        for (int t = wa; t < wb; ++t) key_owner[(size_t)seg[s].g * n_ctx + t]++;
        const int kc = std::max(wa, std::min(wb, pos));
        const int nst = (kc - wa + kpl - 1) / kpl;
        if (nst * kpl < kc - wa) return bad("attention steps miss keys");
      }
      if (kie::attn_owner(m.Hkv, n_ctx, nwg, seg[s].g, seg[s].ta) != w ||
          kie::attn_owner(m.Hkv, n_ctx, nwg, seg[s].g, seg[s].tb - 1) != w)
        return bad("attn_owner disagrees with attn_segments");
    }
  }
  for (int v : key_owner)
    if (v != 1) return bad("attention key covered zero or several times");
  const kie::LdsPlan lp = kie::lds_plan(m, nwg, kie::main_floats(kie::ring_depth_for(m, nwg)));
  // every workgroup's GEMV rows fit the LDS partial sums (and, in the
  // parallel block, the kept O and residual rows)
  for (int k : kinds) {
    for (int w = 0; w < nwg; ++w) {
      int r0, r1;
      kie::gemv_rows_any(m, k, nwg, w, &r0, &r1);
      if (r1 - r0 > lp.rmax) return bad("GEMV rows of a workgroup exceed the LDS partial-sum rows");
      if (k == kie::PH_DOWN && 2 * (r1 - r0) > lp.desc - lp.own) return bad("down rows exceed the LDS row store");
    }
  }
  for (int g = 0; g < m.Hkv; ++g) {
    const int nrec = kie::attn_owner(m.Hkv, n_ctx, nwg, g, n_ctx - 1) - kie::attn_owner(m.Hkv, n_ctx, nwg, g, 0) + 1;
    if (nrec > lp.max_recs) return bad("more attention records per head than the LDS plan holds");
  }
  for (int v : mergers)
    if (v != 1) return bad("a KV head has no merger or several");
  return KIE_OK;
}

int32_t kie_position(const kie_ctx* c) { return c ? c->pos : -1; }

const char* kie_status_string(kie_status s) {
  switch (s) {
    case KIE_OK: return "ok";
    case KIE_ERR_INVALID_ARG: return "invalid argument";
    case KIE_ERR_HIP: return "HIP runtime error";
    case KIE_ERR_CAPACITY: return "KV-cache capacity exceeded";
    case KIE_ERR_STATE: return "context not ready";
    case KIE_ERR_TIMEOUT: return "wait timed out inside the kernel";
    case KIE_ERR_UNSUPPORTED: return "unsupported model shape";
    case KIE_ERR_BAD_TOKEN: return "token id out of range";
    case KIE_ERR_RANGE: return "prefill activation outside the fp16 range";
  }
  return "unknown status";
}

const char* kie_last_error(const kie_ctx* c) { return c ? c->err.c_str() : "null context"; }

void kie_destroy(kie_ctx* c) { delete c; }

}  // extern "C"
