// Layouts and work partitions shared by the host library and the monokernel.
//
// Everything here is plain integer arithmetic: where each packed weight
// matrix lives, where each workspace buffer lives, and which rows / keys each
// workgroup and wave owns.  The host uses the same functions to size buffers
// and to validate a schedule on the CPU; the device uses them to find its work.
#pragma once
#include <stddef.h>
#include <stdint.h>

#if defined(__HIPCC__)
#define KIE_HD __host__ __device__ __forceinline__
#else
#define KIE_HD static inline
#endif

namespace kie {

constexpr int kWave = 64;               // lanes per wavefront (CDNA)
constexpr int kWaves = 8;               // wavefronts per workgroup
constexpr int kThreads = kWave * kWaves;
constexpr int kBlock = 512;             // fp16 elements one wave reads with 16 B per lane (a chunk)
constexpr int kBlock8 = kBlock / 8;     // 16-byte segments per chunk (= lanes)
constexpr int kChunkBytes = kBlock * 2;
constexpr int kPairCols = kBlock / 2;   // columns of each of the two rows in a GEMV chunk
constexpr int kGainRegs = 8;            // RMSNorm gains per thread: d <= kGainRegs * kThreads

enum PhaseKind : int { PH_QKV = 0, PH_ATTN = 1, PH_O = 2, PH_GU = 3, PH_DOWN = 4, PH_LM = 5 };

// phase order inside one layer
//   sequential pre-norm block: QKV ATTN O GU DOWN
//   parallel (lane) block:     QKV GU ATTN O DOWN   (attention and MLP both read x_l)
KIE_HD int phase_kind(int parallel, int j) {
  return parallel ? (j == 0 ? PH_QKV : j == 1 ? PH_GU : j == 2 ? PH_ATTN : j == 3 ? PH_O : PH_DOWN)
                  : j;  // enum order is the sequential order
}

// The parallel block with a residual delay of two or more layers (and its
// inputs staged in LDS, see LdsPlan::pipe) runs software-pipelined: layer
// l's attention is followed by layer l + 1's QKV and gate/up, and only then
// by layer l's O and down projections.
//   QKV_0 GU_0 | ATTN_0 QKV_1 GU_1 O_0 DOWN_0 | ATTN_1 QKV_2 GU_2 O_1 DOWN_1
//   | ... | ATTN_{L-1} O_{L-1} DOWN_{L-1}
// x_{l+1} = x_l + P_{l-delay} is known once the down projection of layer
// l - delay is done, so layer l + 1's QKV and gate/up need nothing from layer
// l; the attention output then has two weight streams of slack before O
// consumes it, and the QKV output three before attention does.  This is the
// one-GPU form of the delayed all-reduce: a layer's partial sum is consumed
// delay layers later, so its exchange hides under other layers' streams.
// phase ph (0 <= ph < 5 L) of a step -> kind and layer
KIE_HD void phase_at(int pipe, int parallel, int L, int ph, int* kind, int* layer) {
  if (!pipe) {
    *kind = phase_kind(parallel, ph % 5);
    *layer = ph / 5;
    return;
  }
  if (ph < 2) {
    *kind = ph == 0 ? PH_QKV : PH_GU;
    *layer = 0;
    return;
  }
  const int j = (ph - 2) / 5 + 1, r = (ph - 2) % 5;  // super-step j = 1 .. L
  if (j == L) {  // the last layer's tail: ATTN O DOWN
    *kind = r == 0 ? PH_ATTN : r == 1 ? PH_O : PH_DOWN;
    *layer = L - 1;
    return;
  }
  *kind = r == 0 ? PH_ATTN : r == 1 ? PH_QKV : r == 2 ? PH_GU : r == 3 ? PH_O : PH_DOWN;
  *layer = (r == 1 || r == 2) ? j : j - 1;
}

struct Dims {
  int L, d, H, Hkv, hd, F, V, G, max_ctx;
  int parallel, delay;
  float eps;
};

// ---------------------------------------------------------------------------
// packed weights (offsets in fp16 elements from the packed base)
//
// Per layer, in order: attn_norm[d], Wqkv[(H+2Hkv)hd][d], Wo[d][H hd],
// mlp_norm[d], Wgu[2F][d], Wd[d][F]; then final_norm[d], Wlm[V][d], E[V][d].
// A matrix with R rows (R even) and K columns is stored as R/2 row pairs,
// each cut into col_blocks(K) blocks of 256 columns; block b of pair p is
// one 1-KB chunk at ((p * col_blocks(K) + b) * 512): 256 columns of row 2p,
// then the same 256 columns of row 2p+1 (columns past K are zero).  A wave
// reading the chunk with 16 bytes per lane gives lanes 0..31 eight columns
// of row 2p each and lanes 32..63 the same columns of row 2p+1, so a lane
// keeps one row's partial sum for all its chunks of the pair and the cross-
// lane sum happens once per pair.  Packed rows are permuted twice:
//   * Wqkv: inside every q and k head, packed row 2i is dim i and row 2i+1 is
//     dim i + hd/2, so the rotate-half RoPE pair of an output sits in one
//     workgroup; v rows are in natural order;
//   * Wgu: packed row 2f is gate row f, row 2f+1 is up row f.
// Each tensor starts on a 256-byte boundary; after the last one come kBlock
// zero elements, so a chunk load that runs past a tensor's end stays inside
// the buffer.  The embedding table keeps stride d (it is gathered, not
// streamed).
// ---------------------------------------------------------------------------
KIE_HD int col_blocks(int K) { return (K + kPairCols - 1) / kPairCols; }
KIE_HD int padded_cols(int K) { return col_blocks(K) * kPairCols; }
KIE_HD uint64_t packed_elems(uint64_t rows, int K) { return rows / 2 * (uint64_t)col_blocks(K) * kBlock; }
// packed offset of element (r, c) of a matrix with K columns
KIE_HD uint64_t packed_at(uint64_t r, int c, int K) {
  return ((r >> 1) * (uint64_t)col_blocks(K) + (uint64_t)(c / kPairCols)) * kBlock + (r & 1) * kPairCols +
         (uint64_t)(c % kPairCols);
}

struct PackLayout {
  uint64_t layer_stride;
  uint64_t attn_norm, wqkv, wo, mlp_norm, wgu, wd;  // within a layer
  uint64_t final_norm, lm_head, embed;              // absolute
  uint64_t total;                                   // elements
};

KIE_HD uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

KIE_HD PackLayout pack_layout(const Dims& m) {
  const uint64_t A = 128;  // 256 bytes
  PackLayout p{};
  uint64_t o = 0;
  const uint64_t d = m.d, qd = (uint64_t)m.H * m.hd, kvd = (uint64_t)m.Hkv * m.hd, F = m.F;
  p.attn_norm = o; o = align_up(o + d, A);
  p.wqkv = o; o = align_up(o + packed_elems(qd + 2 * kvd, m.d), A);
  p.wo = o; o = align_up(o + packed_elems(d, m.H * m.hd), A);
  p.mlp_norm = o; o = align_up(o + d, A);
  p.wgu = o; o = align_up(o + packed_elems(2 * F, m.d), A);
  p.wd = o; o = align_up(o + packed_elems(d, m.F), A);
  p.layer_stride = o;
  o = p.layer_stride * (uint64_t)m.L;
  p.final_norm = o; o = align_up(o + d, A);
  p.lm_head = o; o = align_up(o + packed_elems(m.V, m.d), A);
  p.embed = o; o = align_up(o + (uint64_t)m.V * d, A);
  p.total = o + kBlock;
  return p;
}

// packed row r of the fused QKV matrix -> source row of wq / wk / wv
// (which = 0 q, 1 k, 2 v; src = row inside that matrix)
KIE_HD void qkv_source_row(const Dims& m, int r, int* which, int* src) {
  const int qd = m.H * m.hd, kvd = m.Hkv * m.hd, half = m.hd / 2;
  if (r < qd + kvd) {
    const int base = r < qd ? 0 : qd;
    const int rr = r - base, head = rr / m.hd, j = rr % m.hd;
    *which = r < qd ? 0 : 1;
    *src = head * m.hd + (j & 1) * half + (j >> 1);
  } else {
    *which = 2;
    *src = r - qd - kvd;
  }
}

// ---------------------------------------------------------------------------
// workspace (byte offsets from the workspace base)
//
// "LL" buffers hold 64-bit words: low 32 bits payload (fp32 bits or an int),
// high 32 bits the epoch of the decode step that wrote it.  A reader accepts
// a word only when its epoch is the current step's, so every word carries its
// own readiness and no separate flag or fence is needed for it.
// ---------------------------------------------------------------------------
struct WsLayout {
  uint64_t state;  // int32[64]: [0] status, [1] abort, [2] token state
  uint64_t rope;   // float2 [max_ctx][hd/2]  (cos, sin)
  uint64_t X;      // LL [2L+2][d]     residual stream vectors
  uint64_t Q;      // LL [L][H hd]     rotated, pre-scaled queries
  uint64_t KC;     // LL [L][Hkv hd]   current key (fp16-rounded)
  uint64_t VC;     // LL [L][Hkv hd]   current value (fp16-rounded)
  uint64_t REC;    // LL [L][nwg][2][G][hd+2]  attention partial records
  uint64_t OB;     // LL [L][H hd]     merged attention output
  uint64_t HB;     // LL [L][F]        SwiGLU activations
  uint64_t LMP;    // LL [nwg][2]      per-workgroup (max logit, argmax)
  uint64_t ll_begin, ll_end;
  uint64_t total;
};

KIE_HD WsLayout ws_layout(const Dims& m, int nwg) {
  WsLayout w{};
  uint64_t o = 0;
  const uint64_t A = 256;
  w.state = o; o = align_up(o + 256, A);
  w.rope = o; o = align_up(o + (uint64_t)m.max_ctx * (m.hd / 2) * 8, A);
  w.ll_begin = o;
  w.X = o; o = align_up(o + (uint64_t)(2 * m.L + 2) * m.d * 8, A);
  w.Q = o; o = align_up(o + (uint64_t)m.L * m.H * m.hd * 8, A);
  w.KC = o; o = align_up(o + (uint64_t)m.L * m.Hkv * m.hd * 8, A);
  w.VC = o; o = align_up(o + (uint64_t)m.L * m.Hkv * m.hd * 8, A);
  w.REC = o; o = align_up(o + (uint64_t)m.L * nwg * 2 * m.G * (m.hd + 2) * 8, A);
  w.OB = o; o = align_up(o + (uint64_t)m.L * m.H * m.hd * 8, A);
  w.HB = o; o = align_up(o + (uint64_t)m.L * m.F * 8, A);
  w.LMP = o; o = align_up(o + (uint64_t)nwg * 2 * 8, A);
  w.ll_end = o;
  w.total = o;
  return w;
}

// KV cache: K[l][g][t][hd] then V[l][g][t][hd], fp16, then kBlock elements
// of slack (a chunk of keys that runs past the last row stays in the buffer)
KIE_HD uint64_t kv_offset(const Dims& m, int l, int kv, int g) {
  return (((uint64_t)l * 2 + kv) * m.Hkv + g) * (uint64_t)m.max_ctx * m.hd;
}
KIE_HD uint64_t kv_elems(const Dims& m) { return (uint64_t)m.L * 2 * m.Hkv * (uint64_t)m.max_ctx * m.hd; }
KIE_HD uint64_t kv_alloc_elems(const Dims& m) { return kv_elems(m) + kBlock; }

// ---------------------------------------------------------------------------
// partitions
// ---------------------------------------------------------------------------
// [a, b) = part i of n items split into `parts` contiguous, balanced pieces
KIE_HD void split(int n, int parts, int i, int* a, int* b) {
  *a = (int)(((uint32_t)n * (uint32_t)i) / (uint32_t)parts);
  *b = (int)(((uint32_t)n * (uint32_t)(i + 1)) / (uint32_t)parts);
}
// Split n items over the kWaves waves of a workgroup in contiguous ranges.
// Waves w and w + 4 share a SIMD and the older one, w, wins most issue slots
// while both run, so it gets the larger share: weights (16 + kWaveSkew) and
// (16 - kWaveSkew) sixteenths, so that both finish together.
#ifndef KIE_WAVE_SKEW
#define KIE_WAVE_SKEW 2
#endif
constexpr int kWaveSkew = KIE_WAVE_SKEW;
KIE_HD int wave_cum(int w) { return w <= 4 ? w * (16 + kWaveSkew) : 4 * (16 + kWaveSkew) + (w - 4) * (16 - kWaveSkew); }
KIE_HD void wave_split(int n, int wave, int* a, int* b) {
  *a = (int)(((uint64_t)n * (uint64_t)wave_cum(wave)) / (uint64_t)(16 * kWaves));
  *b = (int)(((uint64_t)n * (uint64_t)wave_cum(wave + 1)) / (uint64_t)(16 * kWaves));
}
// the part that holds item f (0 <= f < n) under split()
KIE_HD int split_owner(int f, int n, int parts) {
  return (int)(((uint32_t)(f + 1) * (uint32_t)parts + (uint32_t)n - 1) / (uint32_t)n) - 1;
}

// GEMV ops: rows, columns and row grouping of each phase (a workgroup owns
// whole row pairs: the packed chunks hold two rows)
struct GemvShape {
  int rows, K, unit_rows;  // unit_rows rows always stay in one workgroup
};
KIE_HD GemvShape gemv_shape(const Dims& m, int kind) {
  switch (kind) {
    case PH_QKV: return {(m.H + 2 * m.Hkv) * m.hd, m.d, 2};
    case PH_O: return {m.d, m.H * m.hd, 2};
    case PH_GU: return {2 * m.F, m.d, 2};
    case PH_DOWN: return {m.d, m.F, 2};
    default: return {m.V, m.d, 2};  // PH_LM
  }
}
KIE_HD int blocks_per_row(int K) { return (K + kBlock - 1) / kBlock; }
KIE_HD int ceil_div(int a, int b) { return (a + b - 1) / b; }

// rows [r0, r1) of op `kind` owned by workgroup wg.  The O projection
// leaves out the attention mergers (the last workgroup of each KV head's
// group, see attn_segments): they combine their head's partial results after
// every other workgroup is done with attention, and the O projection's
// output waits for its slowest producer.  The parallel block keeps the O
// rows with the down projection's (a workgroup adds the two outputs of its
// rows locally), so there both leave the mergers out: their sum is read
// only layers later, and the mergers catch up on their next QKV rows.
KIE_HD void gemv_rows(const Dims& m, int kind, int nwg, int wg, int* r0, int* r1) {
  GemvShape s = gemv_shape(m, kind);
  int a, b;
  if ((kind == PH_O || (m.parallel && kind == PH_DOWN)) && nwg > m.Hkv) {
    const int g = split_owner(wg, nwg, m.Hkv);  // the workgroup's KV head group
    int w0, w1;
    split(nwg, m.Hkv, g, &w0, &w1);
    // wg - g: the workgroup's index among the non-mergers (each earlier group
    // has one merger); a merger gets the empty range where the next one starts
    split(s.rows / s.unit_rows, nwg - m.Hkv, wg - g, &a, &b);
    if (wg == w1 - 1) b = a;
  } else {
    split(s.rows / s.unit_rows, nwg, wg, &a, &b);
  }
  *r0 = a * s.unit_rows;
  *r1 = b * s.unit_rows;
}

// Attention mergers per KV head group.  With more than two query heads per
// KV head each query head has a merger of its own, the last G workgroups of
// the group (workgroup w1 - 1 - h merges head h), when every group has that
// many: one merger would read G heads of every record in the group, and a
// workgroup's record poll is bound by its own memory requests.  Otherwise
// the group's last workgroup merges all of its heads.
KIE_HD int attn_mergers(const Dims& m, int nwg) { return (m.G > 2 && nwg / m.Hkv >= m.G) ? m.G : 1; }
// gemv_rows with nm mergers per group left out of the O (and, in the
// parallel block, the down) projection
KIE_HD void gemv_rows_nm(const Dims& m, int kind, int nwg, int wg, int nm, int* r0, int* r1) {
  GemvShape s = gemv_shape(m, kind);
  int a, b;
  if ((kind == PH_O || (m.parallel && kind == PH_DOWN)) && nwg > m.Hkv * nm) {
    const int g = split_owner(wg, nwg, m.Hkv);
    int w0, w1;
    split(nwg, m.Hkv, g, &w0, &w1);
    // index among the non-mergers (nm per earlier group); a merger gets the
    // empty range where the next non-merger starts
    const int first = w1 - nm;
    split(s.rows / s.unit_rows, nwg - m.Hkv * nm, (wg < first ? wg : first) - g * nm, &a, &b);
    if (wg >= first) b = a;
  } else {
    split(s.rows / s.unit_rows, nwg, wg, &a, &b);
  }
  *r0 = a * s.unit_rows;
  *r1 = b * s.unit_rows;
}
// the rows of any shape (host side, and the kernels with more than two
// query heads per KV head)
KIE_HD void gemv_rows_any(const Dims& m, int kind, int nwg, int wg, int* r0, int* r1) {
  const int nm = attn_mergers(m, nwg);
  if (nm > 1) {
    gemv_rows_nm(m, kind, nwg, wg, nm, r0, r1);
  } else {
    gemv_rows(m, kind, nwg, wg, r0, r1);
  }
}

// The workgroup's row pairs are one contiguous stretch of nrows / 2 *
// col_blocks(K) chunks; wave w takes chunks [c0, c1).
KIE_HD int gemv_chunks(int nrows, int K) { return nrows / 2 * col_blocks(K); }
KIE_HD void gemv_wave_chunks(int nrows, int K, int wave, int* c0, int* c1) {
  wave_split(gemv_chunks(nrows, K), wave, c0, c1);
}

// attention: the workgroups are cut into Hkv contiguous groups (split), one
// per KV head, and the n_ctx keys of head g into one contiguous range per
// workgroup of its group, so no workgroup meets two heads and every one that
// has keys has exactly one "segment"; each segment is cut into kWaves
// contiguous key ranges, one per wave (wave_split).  The last workgroup of a
// group holds the newest key and merges the group's partial results.
struct AttnSeg {
  int g;       // KV head
  int ta, tb;  // workgroup's keys [ta, tb) of head g
};
KIE_HD int attn_head(int Hkv, int nwg, int wg) { return split_owner(wg, nwg, Hkv); }
KIE_HD int attn_segments(int Hkv, int n_ctx, int nwg, int wg, AttnSeg* seg) {
  const int g = attn_head(Hkv, nwg, wg);
  int w0, w1, ta, tb;
  split(nwg, Hkv, g, &w0, &w1);
  split(n_ctx, w1 - w0, wg - w0, &ta, &tb);
  if (ta >= tb) return 0;
  seg[0].g = g;
  seg[0].ta = ta;
  seg[0].tb = tb;
  return 1;
}

// workgroup that holds key t of head g
KIE_HD int attn_owner(int Hkv, int n_ctx, int nwg, int g, int t) {
  int w0, w1;
  split(nwg, Hkv, g, &w0, &w1);
  return w0 + split_owner(t, n_ctx, w1 - w0);
}

// lanes per key (16 bytes of a key row per lane) and keys per wave load
KIE_HD int attn_lpk(int hd) { return hd / 8; }
KIE_HD int attn_kpl(int hd) { return kWave / (hd / 8); }

// per-wave work descriptors kept in LDS (ints):
//   GEMV kind k (0 QKV, 1 O, 2 GU, 3 DOWN, 4 LM): 8 ints at wave*kWaveDesc + 8k
//     {offset lo, offset hi (elements from the layer base to the wave's first
//      chunk), chunks, first row, first column, row stride, 0, 0}
//   attention (this step): 12 ints at wave*kWaveDesc + 52
//     {g0, ka0, kc0, nst0, pos0, g1, ka1, kc1, nst1, pos1, nseg, merge_g}
//   workgroup rows per GEMV kind: 2 ints at kWaves*kWaveDesc + 2k {r0, nrows}
constexpr int kWaveDesc = 64;
constexpr int kConsumerAttn = 52;
constexpr int kDescInts = kWaves * kWaveDesc + 16;
// The library holds the kernel built for two ring depths (LDS slots per
// wave): kRingDeep for the sequential block wherever its LDS plan fits
// beside the deeper ring (more of the next phases' weights in flight while
// a wave waits on an exchange: cfg1 -3.8 %, cfg2 -0.4 % per token), and
// kRingBase otherwise.  The lane block keeps the base ring: a deeper one
// leaves no LDS for its staged inputs.
constexpr int kRingBase = 8, kRingDeep = 10;
#ifndef KIE_RING_DEPTH
#define KIE_RING_DEPTH 8
#endif
constexpr int kRingDepth = KIE_RING_DEPTH;  // the depth of the kernel being compiled
// LDS of one workgroup: the ring (kWaves x depth KB), a small block of
// shared scalars, and one static array of main_floats(depth) floats for
// everything else; a model whose LdsPlan needs more is rejected by the host
constexpr int kLdsBytes = 160 * 1024;
constexpr int kSharedReserve = 256;
KIE_HD constexpr int main_floats(int depth) { return (kLdsBytes - depth * kWaves * kChunkBytes - kSharedReserve) / 4; }
constexpr int kMainFloats = main_floats(kRingDepth);

// phase slots of one step in the LDS trace buffer: 5 per layer, the LM
// head, the end of the step
KIE_HD int trace_slots(int L) { return 5 * L + 2; }

// LDS plan (in floats)
struct LdsPlan {
  int xraw, big, gemv_xs, gemv_part, attn_wrec, attn_ml, attn_qkv, own, desc, trace;
  // parallel block: the down projection's input (two planes, kmax floats) and
  // the next layer's two RMSNorm gain vectors (whole 1-KB chunks: attention
  // gains at half 0, MLP gains at half align(d, 512)), both fetched in
  // the O prologue; -1 when they do not fit
  int hb, gst;
  // 1: the parallel block runs in the pipelined phase order (phase_at).  It
  // needs the staged inputs above (two or fewer query heads per KV head) and
  // a residual delay of at least two layers: the O prologue of layer l then
  // stages x_{l+2}, which the down projection of layer l + 2 - delay - 1 <= l - 1
  // has already published.
  int pipe;
  int total_floats;
  int kmax, rmax, max_recs;
};
KIE_HD int imax(int a, int b) { return a > b ? a : b; }
// the plan for a kernel whose main LDS array holds `budget` floats
KIE_HD LdsPlan lds_plan(const Dims& m, int nwg, int budget) {
  LdsPlan p{};
  // GEMV input: two planes of kmax/2 floats (elements 8g..8g+3 at plane 0,
  // 8g+4..8g+7 at plane 1, position 4g), covering padded_cols(K) elements
  int kmax = imax(imax(imax(padded_cols(m.d), padded_cols(m.H * m.hd)), padded_cols(m.F)), 2 * nwg);
  kmax = (int)align_up((uint64_t)kmax, kBlock);
  // the most GEMV rows any workgroup owns (the splits are uneven), and the
  // most rows of the down projection (the parallel block keeps those)
  int rmax = 0, dmax = 0;
  for (int k = 0; k <= PH_LM; ++k) {
    if (k == PH_ATTN) continue;
    for (int w = 0; w < nwg; ++w) {
      int r0, r1;
      gemv_rows_any(m, k, nwg, w, &r0, &r1);
      rmax = imax(rmax, r1 - r0);
      if (k == PH_DOWN) dmax = imax(dmax, r1 - r0);
    }
  }
  // records merged for one head: workgroups meeting that head
  const int max_recs = (nwg + m.Hkv - 1) / m.Hkv + 2;
  p.kmax = kmax;
  p.rmax = rmax;
  p.max_recs = max_recs;
  int o = 0;
  p.xraw = o; o += (int)align_up((uint64_t)m.d, 64);
  p.big = o;
  p.gemv_xs = o;
  p.gemv_part = o + kmax;
  const int gemv_sz = kmax + (int)align_up((uint64_t)rmax * kWaves, 64);
  // attention: per-wave records (2 segments x kWaves), later reused by the
  // merger for the records of every workgroup that met its head, then
  // 8 floats per record (its weight for each query head, its segment), then
  // per segment the G query heads and the key and value at the current
  // position
  const int wrec_sz = imax(2 * kWaves * m.G * (m.hd + 2), max_recs * m.G * (m.hd + 2));
  p.attn_wrec = o;
  p.attn_ml = o + wrec_sz;
  p.attn_qkv = p.attn_ml + max_recs * 8;
  const int attn_sz = wrec_sz + max_recs * 8 + 2 * (m.G + 2) * m.hd;
  o += (int)align_up((uint64_t)imax(gemv_sz, attn_sz), 64);
  p.own = o; o += (int)align_up((uint64_t)2 * dmax, 64);
  p.desc = o; o += kDescInts;
  p.hb = -1;
  p.gst = -1;
  p.pipe = 0;
  if (m.parallel) {
    const int hb = (int)align_up((uint64_t)o, 64);
    const int gst = hb + kmax;
    const int end = gst + (int)align_up((uint64_t)m.d, kBlock);  // 2 x align(d, 512) halves
    if (end <= budget) {
      p.hb = hb;
      p.gst = gst;
      p.pipe = m.G <= 2 && m.delay >= 2;
      o = end;
    }
  }
  // phase trace of one step (32-bit stamps, written out at the step's end),
  // when it fits; otherwise stamps go straight to memory
  p.trace = -1;
  if (o + trace_slots(m.L) * 4 <= budget) {
    p.trace = o;
    o += trace_slots(m.L) * 4;
  }
  p.total_floats = o;
  return p;
}

// the ring depth the host runs a model with (kRingDeep or kRingBase)
KIE_HD int ring_depth_for(const Dims& m, int nwg) {
  if (m.parallel) return kRingBase;
  const int deep = main_floats(kRingDeep);
  return lds_plan(m, nwg, deep).total_floats <= deep ? kRingDeep : kRingBase;
}

// arguments of one monokernel launch
struct KParams {
  Dims m;
  PackLayout pl;
  WsLayout wl;
  LdsPlan lp;
  const uint16_t* W;  // packed weights
  uint16_t* kv;       // KV cache
  uint8_t* ws;        // workspace
  const int32_t* forced;  // [n_steps] or null
  int32_t* out;           // [n_steps] or null
  float* logits;          // [n_steps][V] or null
  int n_steps, pos0;
  int lm_mode;            // 0: LM head every step; 1: last step only; 2: never
  int first_from_state;   // 1: step 0 reads the token state word
  uint32_t epoch0;        // epoch of step 0
  uint64_t timeout_ticks; // wall-clock ticks a single wait may take
  uint32_t debug_flags;
  // optional phase trace: for steps < trace_steps, workgroup wg's thread 0
  // writes 4 wall-clock stamps per phase (start, input ready, stream done,
  // end) at trace[((step * kTracePhases + phase) * nwg + wg) * 4]
  uint64_t* trace;
  int trace_steps;
  // stochastic LM-head sampling (sample != 0): the token is the argmax of
  // logits * inv_temp + Gumbel noise from Philox4x32-10 keyed by
  // (seed_lo, seed_hi) at counter (row, position, 0, 0)
  int sample;
  float inv_temp;
  uint32_t seed_lo, seed_hi;
};
constexpr int kTracePhases = 5 * 64 + 2;  // up to 64 layers, LM, step end

// Batched prefill of prompt tokens [0, C) of one chunk (all but the prompt's
// last token go this way; the last one runs through the decode kernel).  The
// chunk's activations live in caller scratch, fp32, token-major:
//   X  [C][d]                residual stream
//   Y  [C][max(d, F)]        RMSNorm output, then the SwiGLU activations
//   Gb [C][max(qd+2kvd, 2F)] QKV or gate/up GEMM output (packed row order)
//   Qn [C][qd]               rotated queries, scaled by log2(e)/sqrt(hd)
//   Ao [C][qd]               attention output (natural head-major order)
// and for the lane-structured block P [C][d] and R [delay + 2][C][d]
// (X then holds x_0, the embedding).
struct PrefillArgs {
  Dims m;
  PackLayout pl;
  const uint16_t* W;     // packed weights
  uint16_t* kv;          // KV cache
  const float2* rope;    // [max_ctx][hd/2] (cos, sin)
  int32_t* state;        // device status words (bad token -> DEV_BAD_TOKEN, fp16 range -> DEV_RANGE)
  const int32_t* tokens; // [C] device ids of this chunk
  int C, pos0;
  float* scratch;
};
KIE_HD int pf_ycols(const Dims& m) { return m.d > m.F ? m.d : m.F; }
KIE_HD int pf_gcols(const Dims& m) {
  const int qkv = (m.H + 2 * m.Hkv) * m.hd;
  return qkv > 2 * m.F ? qkv : 2 * m.F;
}
// fp32 scratch floats per prompt token of a chunk; the lane-structured
// block adds its partial sums P [C][d] and delay + 2 residual states
// R_l = x_0 + P_0 + .. + P_l [C][d] (layer l reads R_{l - delay - 1})
KIE_HD uint64_t pf_floats_per_token(const Dims& m) {
  return (uint64_t)m.d + pf_ycols(m) + pf_gcols(m) + 2ull * m.H * m.hd +
         (m.parallel ? (uint64_t)(m.delay + 3) * m.d : 0ull);
}

// the no-allocation batched prefill's scratch: one array of this many bytes
// per GPU, held until the process ends; devices numbered below kMaxDevices
constexpr uint64_t kNoAllocScratchBytes = 64ull << 20;
constexpr int kMaxDevices = 64;

enum DebugFlags : uint32_t {
  DBG_WAIT_NEVER = 1u,  // workgroup 0 waits on a word no one writes (timeout test)
  DBG_JITTER = 2u,      // every wave sleeps a pseudo-random time at every phase start
};

enum DeviceStatus : int32_t { DEV_OK = 0, DEV_TIMEOUT = 1, DEV_BAD_TOKEN = 2, DEV_RANGE = 3 };

}  // namespace kie
