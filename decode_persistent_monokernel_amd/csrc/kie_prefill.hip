// Batched prefill: the prompt's tokens (all but the last) pushed through the
// layers a chunk of C tokens at a time, with the weight GEMMs on the matrix
// cores.  The pages' monokernel runs prefill on the GPU as well (Kog
// explainer, "Monokernel" section); batching the prompt turns its GEMVs into
// dense [C x K] x [K x N] products, so each weight is read once per chunk
// instead of once per token.
//
// Arithmetic matches the decode kernel's to fp32 accuracy: fp32 activations
// (in the weight GEMMs carried as fp16 hi + lo pairs on the fp16 matrix
// cores), fp16 weights, fp32 accumulation, the same RMSNorm, RoPE, fp16
// rounding of cached K and V, exp2-domain softmax and SwiGLU formulas.  Only
// summation orders (and the ~2^-22 split error) differ.
//
// Kernels, launched in stream order per chunk and layer:
//   embed -> [rmsnorm -> gemm(QKV) -> rope_kv -> attention -> gemm(O, +X)
//             -> rmsnorm -> gemm(gate/up) -> swiglu -> gemm(down, +X)] x L
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "kie_layout.h"

namespace kie {
namespace pf {

typedef float f16v __attribute__((ext_vector_type(16)));

constexpr int kRowThreads = 256;

__device__ __forceinline__ float h2f(uint16_t u) { return __half2float(__ushort_as_half(u)); }

// fp32 values as fp16 pairs for the fp16 matrix cores: hi = fp16(x) and
// lo = fp16((x - hi) * 2^11), so that x = hi + lo * 2^-11 to about 2^-22
// relative.  The remainder x - hi is scaled by the power of two 2^11 (exact)
// before its rounding: unscaled it falls below fp16's normal range whenever
// |x| < 2^-3, and the matrix cores would see a subnormal (or flushed)
// operand.  Products of lo go to their own fp32 accumulator, which is scaled
// back by 2^-11 once, at the end.  Both parts stay normal for |x| >= 2^-14.
typedef _Float16 h4v __attribute__((ext_vector_type(4)));
constexpr float kLoScale = 2048.0f, kLoUnscale = 1.0f / 2048.0f;
__device__ __forceinline__ void split4(const float4 x, h4v& hi, h4v& lo) {
  const float v[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    hi[i] = (_Float16)v[i];
    lo[i] = (_Float16)((v[i] - (float)hi[i]) * kLoScale);
  }
}

__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) t += red[i];
  __syncthreads();
  return t;
}

// X[m][:] = E[token m]; an id outside [0, V) reads row 0 and latches
// DEV_BAD_TOKEN in the status word, as in the decode kernel
__global__ void __launch_bounds__(kRowThreads) embed(float* X, const uint16_t* W, uint64_t embed_off,
                                                     const int32_t* tok, int d, int V, int32_t* state) {
  const int m = blockIdx.x;
  int t = tok[m];
  if (t < 0 || t >= V) {
    if (threadIdx.x == 0) atomicCAS(&state[0], 0, (int)DEV_BAD_TOKEN);
    t = 0;
  }
  const uint16_t* e = W + embed_off + (uint64_t)t * d;
  for (int i = threadIdx.x; i < d; i += blockDim.x) X[(uint64_t)m * d + i] = h2f(e[i]);
}

// Y[m][:] = g * x / sqrt(mean(x^2) + eps)
__global__ void __launch_bounds__(kRowThreads) rmsnorm(float* Y, int ldy, const float* X, int d,
                                                       const uint16_t* g, float eps) {
  __shared__ float red[kRowThreads / 64];
  const int m = blockIdx.x;
  const float* x = X + (uint64_t)m * d;
  float ss = 0.f;
  for (int i = threadIdx.x; i < d; i += blockDim.x) ss += x[i] * x[i];
  const float tot = block_sum(ss, red);
  const float inv = 1.0f / sqrtf(tot / (float)d + eps);
  for (int i = threadIdx.x; i < d; i += blockDim.x) Y[(uint64_t)m * ldy + i] = x[i] * inv * h2f(g[i]);
}

// Out[m][n] (+)= sum_k A[m][k] * W[n][k] for m < M, n < N.  W is a packed
// matrix: row pairs, each cut into 256-column blocks of one 1 KB chunk (256
// columns of row 2p, then the same columns of row 2p+1, zero past K).
// Tile 64 (m) x 128 (n) x 64 (k) per workgroup of 4 waves; wave w owns
// columns n0 + 32w .. +32 and both 32-row halves, two 32x32 accumulators.
// The next k tile is fetched into registers while the current one is
// multiplied from LDS (double-buffered).
constexpr int BM = 64, BN = 128, BK = 64;

// The product runs on the fp16 matrix cores to fp32 accuracy: each fp32
// activation a is split into hi and a scaled lo (split4: a = hi + lo 2^-11
// to about 2^-22 relative), and the weights are fp16 already; hi * W and
// lo * W accumulate in two fp32 accumulators (v_mfma_f32_32x32x16_f16, two
// per k-step of 16, operands read from LDS 16 bytes per lane), added as
// hi + 2^-11 lo at the end.  The split happens
// once, when a tile is staged in LDS.  LDS rows hold 72 halves (144 bytes, a
// multiple of 16 for the 16-byte reads).
typedef _Float16 h8v __attribute__((ext_vector_type(8)));
constexpr int HP = BK + 8;

template <bool ADD>
__global__ void __launch_bounds__(256) gemm16(float* Out, int ldo, const float* A, int lda, const uint16_t* Wm,
                                              int M, int N, int K, int32_t* state) {
  __shared__ _Float16 Ah[2][BM][HP];
  __shared__ _Float16 Al[2][BM][HP];
  __shared__ uint16_t Bh[2][BN][HP];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int nkt = (K + BK - 1) / BK;
  const int cb = col_blocks(K);
  // loads of this thread: A rows ar and ar + 32, columns ak + 32 c .. +3
  // (c < 2); B row bn (packed), columns bk .. bk + 31
  const int ar = tid >> 3, ak = (tid & 7) * 4;
  const int bn = tid >> 1, bk = (tid & 1) * 32;
  float4 ra[4];
  uint4 rb[4];
  // an activation fp16 cannot carry (|a| > 65504, inf or NaN) is latched as
  // DEV_RANGE in the status word instead of reaching the KV cache unnoticed
  bool out_of_range = false;
  auto fetch = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int m = m0 + ar + 32 * (h & 1), k = k0 + ak + 32 * (h >> 1);
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (m < M) {
        const float* a = A + (uint64_t)m * lda + k;
        if (k + 3 < K) {
          v = *(const float4*)a;
        } else {
          v.x = k < K ? a[0] : 0.f;
          v.y = k + 1 < K ? a[1] : 0.f;
          v.z = k + 2 < K ? a[2] : 0.f;
          v.w = 0.f;
        }
      }
      ra[h] = v;
    }
    const int n = n0 + bn, k = k0 + bk;  // k + 31 < 256 * cb: the padded row holds it
    if (n < N) {
      const uint16_t* w = Wm + ((uint64_t)(n >> 1) * cb + (k >> 8)) * 512 + (n & 1) * 256 + (k & 255);
#pragma unroll
      for (int i = 0; i < 4; ++i) rb[i] = *(const uint4*)(w + 8 * i);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) rb[i] = make_uint4(0, 0, 0, 0);
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      h4v hi, lo;
      out_of_range |= !(fmaxf(fmaxf(fabsf(ra[h].x), fabsf(ra[h].y)), fmaxf(fabsf(ra[h].z), fabsf(ra[h].w))) <= 65504.f);
      split4(ra[h], hi, lo);
      *(h4v*)&Ah[buf][ar + 32 * (h & 1)][ak + 32 * (h >> 1)] = hi;
      *(h4v*)&Al[buf][ar + 32 * (h & 1)][ak + 32 * (h >> 1)] = lo;
    }
    uint2* d = (uint2*)&Bh[buf][bn][bk];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      d[2 * i] = make_uint2(rb[i].x, rb[i].y);
      d[2 * i + 1] = make_uint2(rb[i].z, rb[i].w);
    }
  };
  f16v acc[2], accl[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc[i][r] = 0.f;
      accl[i][r] = 0.f;
    }
  fetch(0);
  stash(0);
  __syncthreads();
  const int li = lane & 31, lk = lane >> 5;
  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nkt) fetch(kt + 1);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      // operands: lane l holds row (or column) l % 32, k = kk + 8 (l / 32) .. +7
      const int kq = kk + 8 * lk;
      const h8v b = *(const h8v*)&Bh[buf][wave * 32 + li][kq];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const h8v ah = *(const h8v*)&Ah[buf][32 * i + li][kq];
        const h8v al = *(const h8v*)&Al[buf][32 * i + li][kq];
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, b, acc[i], 0, 0, 0);
        accl[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, b, accl[i], 0, 0, 0);
      }
    }
    if (kt + 1 < nkt) stash(buf ^ 1);
    __syncthreads();
  }
  if (out_of_range) atomicCAS(state, 0, (int)DEV_RANGE);
  // accumulator layout of a 32x32 tile: lane l, element r holds row
  // 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32
  const int n = n0 + wave * 32 + li;
  if (n >= N) return;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + 32 * i + 8 * (r >> 2) + 4 * lk + (r & 3);
      if (m < M) {
        float* o = Out + (uint64_t)m * ldo + n;
        const float y = __builtin_fmaf(accl[i][r], kLoUnscale, acc[i][r]);
        *o = ADD ? *o + y : y;
      }
    }
}

// The QKV output of token m (packed row order: row pairs are RoPE partners
// (i, i + hd/2) of a q or k head, or consecutive value dims): rotate q and k
// at position pos0 + m, write q scaled by log2(e)/sqrt(hd) in natural order
// to Qn, and k and v rounded to fp16 into the cache -- the decode kernel's
// QKV epilogue, one token per workgroup.
__global__ void __launch_bounds__(kRowThreads) rope_kv(float* Qn, const float* Gb, int ldg, uint16_t* kv,
                                                       const float2* rope, Dims m, int l, int pos0) {
  const int mq = blockIdx.x, pos = pos0 + mq;
  const int hd = m.hd, qd = m.H * hd, kvd = m.Hkv * hd;
  const float qscale = 1.4426950408889634f / sqrtf((float)hd);
  const float* y = Gb + (uint64_t)mq * ldg;
  for (int t = threadIdx.x; t < (qd + 2 * kvd) / 2; t += blockDim.x) {
    const int rr = 2 * t;
    const float y0 = y[rr], y1 = y[rr + 1];
    if (rr < qd + kvd) {
      const bool isq = rr < qd;
      const int base = isq ? 0 : qd;
      const int head = (rr - base) / hd;
      const int i = ((rr - base) % hd) >> 1;
      const float2 cs = rope[(uint64_t)pos * (hd / 2) + i];
      const float a = y0 * cs.x - y1 * cs.y;
      const float b = y0 * cs.y + y1 * cs.x;
      if (isq) {
        float* q = Qn + (uint64_t)mq * qd + (uint64_t)head * hd;
        q[i] = a * qscale;
        q[i + hd / 2] = b * qscale;
      } else {
        uint16_t* kc = kv + kv_offset(m, l, 0, head) + (uint64_t)pos * hd;
        kc[i] = __half_as_ushort(__float2half_rn(a));
        kc[i + hd / 2] = __half_as_ushort(__float2half_rn(b));
      }
    } else {
      const int jv = rr - qd - kvd;
      const int head = jv / hd, dd = jv % hd;
      uint16_t* vc = kv + kv_offset(m, l, 1, head) + (uint64_t)pos * hd;
      vc[dd] = __half_as_ushort(__float2half_rn(y0));
      vc[dd + 1] = __half_as_ushort(__float2half_rn(y1));
    }
  }
}

// Causal attention of the chunk's queries over the cache: one wave per
// (query token, query head).  Keys go 64 at a time, one per lane (its score
// is the lane's own dot product); an online softmax in the log2 domain
// rescales the running sums once per block; each lane accumulates the output
// dims lane, lane + 64, ... (at most kMaxDims of them).
constexpr int kMaxDims = 8;  // hd <= 512

__global__ void __launch_bounds__(256) attention(float* Ao, const float* Qn, const uint16_t* kv, Dims m, int l,
                                                 int pos0, int C) {
  extern __shared__ float qsh[];  // [4][hd]
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + wave;
  const int hd = m.hd, H = m.H, qd = H * hd;
  const int mq = gw / H, h = gw % H;
  float* q = qsh + wave * hd;
  if (mq < C) {
    for (int i = lane; i < hd; i += 64) q[i] = Qn[(uint64_t)mq * qd + (uint64_t)h * hd + i];
  }
  __syncthreads();
  if (mq >= C) return;
  const int g = h / m.G;
  const int nkeys = pos0 + mq + 1;
  const uint16_t* K = kv + kv_offset(m, l, 0, g);
  const uint16_t* V = kv + kv_offset(m, l, 1, g);
  float acc[kMaxDims];
#pragma unroll
  for (int e = 0; e < kMaxDims; ++e) acc[e] = 0.f;
  float mrun = -INFINITY, lrun = 0.f;
  for (int j0 = 0; j0 < nkeys; j0 += 64) {
    const int j = j0 + lane;
    float s = -INFINITY;
    if (j < nkeys) {
      const uint16_t* kr = K + (uint64_t)j * hd;
      float t = 0.f;
      for (int d0 = 0; d0 < hd; d0 += 8) {
        const uint4 w = *(const uint4*)(kr + d0);
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          t = __builtin_fmaf(h2f((uint16_t)(ww[e] & 0xFFFF)), q[d0 + 2 * e], t);
          t = __builtin_fmaf(h2f((uint16_t)(ww[e] >> 16)), q[d0 + 2 * e + 1], t);
        }
      }
      s = t;
    }
    float bm = s;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) bm = fmaxf(bm, __shfl_xor(bm, off));
    const float mn = fmaxf(mrun, bm);
    const float scale = mrun == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrun - mn);
    const float p = s == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s - mn);
    float ps = p;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ps += __shfl_xor(ps, off);
    lrun = lrun * scale + ps;
    mrun = mn;
#pragma unroll
    for (int e = 0; e < kMaxDims; ++e) acc[e] *= scale;
    const int nb = nkeys - j0 < 64 ? nkeys - j0 : 64;
    for (int jj = 0; jj < nb; ++jj) {
      const float pj = __shfl(p, jj);
      const uint16_t* vr = V + (uint64_t)(j0 + jj) * hd;
#pragma unroll
      for (int e = 0; e < kMaxDims; ++e) {
        const int dd = lane + 64 * e;
        if (dd < hd) acc[e] = __builtin_fmaf(pj, h2f(vr[dd]), acc[e]);
      }
    }
  }
  float* o = Ao + (uint64_t)mq * qd + (uint64_t)h * hd;
#pragma unroll
  for (int e = 0; e < kMaxDims; ++e) {
    const int dd = lane + 64 * e;
    if (dd < hd) o[dd] = acc[e] / lrun;
  }
}

// Causal attention on the matrix cores (flash-attention order): a workgroup
// takes 64 query tokens of one head, wave w the 16 tokens 16w .. 16w+15.  Key
// blocks of 64 are staged in LDS as the cache holds them, fp16 (K as is, V
// transposed; zero past the last key) and shared by the four waves.  Per
// block, with v_mfma_f32_16x16x16f16: S = Q K^T (16 x 64 per wave, the
// log2-domain scores), masked above the diagonal; a row-wise online softmax
// (max and sum over the 16 lanes holding a row's columns, DPP); P goes through
// LDS into the A-operand layout; O += P V.  Q and P enter the products as
// fp16 hi + lo pairs (split4), so both products keep fp32 accuracy, like the
// decode kernel's attention.
// For hd a multiple of 16 and at most 128 (larger heads use `attention`).
typedef float f4v __attribute__((ext_vector_type(4)));
constexpr int FQ = 64, FK = 64;  // query tokens and keys per block

__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
  return v;
}
__device__ __forceinline__ float row16_add(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
  return v;
}

template <int HD>
__global__ void __launch_bounds__(256) attention_mfma(float* Ao, const float* Qn, const uint16_t* kv, Dims m, int l,
                                                      int pos0, int C) {
  constexpr int KS = HD + 4;  // K row stride (halves): a fragment's 16 rows start in different banks
  constexpr int VT = FK + 4;  // transposed V row stride (halves)
  constexpr int PS = FK + 4;  // P row stride (floats)
  constexpr int NS = HD / 16;  // k-steps of Q K^T
  constexpr int NU = HD / 16;  // 16-wide output column tiles
  __shared__ uint16_t Ks[FK * KS];  // K[key][dim], fp16 as stored
  __shared__ uint16_t Vt[HD * VT];  // V[key][dim] transposed: Vt[dim][key]
  __shared__ float Ps[4][16 * PS];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lq = lane >> 4;
  const int qb = blockIdx.x, h = blockIdx.y;
  const int H = m.H, qd = H * HD, g = h / m.G;
  const int t0 = qb * FQ + wave * 16;  // this wave's first token in the chunk
  // Q fragments: lane holds Q[token t0 + lr][dims 16 s + 4 lq .. +3], split
  // into fp16 hi and lo parts
  h4v qh[NS], ql[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int t = t0 + lr;
    float4 q = make_float4(0.f, 0.f, 0.f, 0.f);
    if (t < C) q = *(const float4*)(Qn + (uint64_t)t * qd + (uint64_t)h * HD + 16 * s + 4 * lq);
    split4(q, qh[s], ql[s]);
  }
  f4v acc[NU], accl[NU];  // P V of the hi and the (scaled) lo parts of P
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    acc[u] = f4v{0.f, 0.f, 0.f, 0.f};
    accl[u] = f4v{0.f, 0.f, 0.f, 0.f};
  }
  float mrow[4], lrow[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    mrow[r] = -INFINITY;
    lrow[r] = 0.f;
  }
  // query positions of the rows this lane holds in the S and O layouts
  int qpos[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) qpos[r] = pos0 + t0 + 4 * lq + r;
  const int last_tok = min(C, qb * FQ + FQ) - 1;
  const int nkeys = pos0 + last_tok + 1;  // keys the block's last query sees
  const uint16_t* K = kv + kv_offset(m, l, 0, g);
  const uint16_t* V = kv + kv_offset(m, l, 1, g);
  float* P = Ps[wave];
  for (int k0 = 0; k0 < nkeys; k0 += FK) {
    __syncthreads();  // the previous block's K, V are consumed
    // stage keys k0 .. k0+63: 8 halves per thread and pass
    for (int i = tid; i < FK * HD / 8; i += 256) {
      const int key = i / (HD / 8), c = (i % (HD / 8)) * 8;
      uint4 kw = make_uint4(0, 0, 0, 0), vw = make_uint4(0, 0, 0, 0);
      if (k0 + key < nkeys) {
        kw = *(const uint4*)(K + (uint64_t)(k0 + key) * HD + c);
        vw = *(const uint4*)(V + (uint64_t)(k0 + key) * HD + c);
      }
      uint2* kd = (uint2*)(Ks + key * KS + c);
      kd[0] = make_uint2(kw.x, kw.y);
      kd[1] = make_uint2(kw.z, kw.w);
      const uint32_t vv[4] = {vw.x, vw.y, vw.z, vw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Vt[(c + 2 * e) * VT + key] = (uint16_t)(vv[e] & 0xFFFF);
        Vt[(c + 2 * e + 1) * VT + key] = (uint16_t)(vv[e] >> 16);
      }
    }
    __syncthreads();
    // S = Q K^T for the 4 key tiles of 16 (B operand: lane holds key
    // 16 kt + lr, dims 16 s + 4 lq .. +3)
    f4v sc[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      sc[kt] = f4v{0.f, 0.f, 0.f, 0.f};
      f4v scl = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const h4v kb = *(const h4v*)(Ks + (kt * 16 + lr) * KS + 16 * s + 4 * lq);
        sc[kt] = __builtin_amdgcn_mfma_f32_16x16x16f16(qh[s], kb, sc[kt], 0, 0, 0);
        scl = __builtin_amdgcn_mfma_f32_16x16x16f16(ql[s], kb, scl, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[kt][r] = __builtin_fmaf(scl[r], kLoUnscale, sc[kt][r]);
    }
    // mask (key position > query position, or past the keys) and row maxima
    float bm[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int kpos = k0 + kt * 16 + lr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (kpos > qpos[r]) sc[kt][r] = -INFINITY;
        bm[r] = fmaxf(bm[r], sc[kt][r]);
      }
    }
    float scale[4], mn[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      bm[r] = row16_max(bm[r]);
      mn[r] = fmaxf(mrow[r], bm[r]);
      scale[r] = mn[r] == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(mrow[r] - mn[r]);
    }
    float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pv = sc[kt][r] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc[kt][r] - mn[r]);
        rs[r] += pv;
        P[(4 * lq + r) * PS + kt * 16 + lr] = pv;  // P[row][key]
      }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      lrow[r] = lrow[r] * scale[r] + row16_add(rs[r]);
      mrow[r] = mn[r];
    }
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        acc[u][r] *= scale[r];
        accl[u][r] *= scale[r];
      }
    // the wave's own P tile: its LDS writes must land before its reads
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    // O += P V: A = P[row lr][keys 16 s + 4 lq .. +3] (split into hi and lo),
    // B = V[keys 16 s + 4 lq .. +3][dim 16 u + lr]
#pragma unroll
    for (int s = 0; s < FK / 16; ++s) {
      h4v ph, pl;
      split4(*(const float4*)(P + lr * PS + 16 * s + 4 * lq), ph, pl);
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const h4v vb = *(const h4v*)(Vt + (16 * u + lr) * VT + 16 * s + 4 * lq);
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x16f16(ph, vb, acc[u], 0, 0, 0);
        accl[u] = __builtin_amdgcn_mfma_f32_16x16x16f16(pl, vb, accl[u], 0, 0, 0);
      }
    }
  }
  // O = acc / l, rows 4 lq + r, columns 16u + lr
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = t0 + 4 * lq + r;
    if (t >= C) continue;
    float* o = Ao + (uint64_t)t * qd + (uint64_t)h * HD;
    const float inv = 1.0f / lrow[r];
#pragma unroll
    for (int u = 0; u < NU; ++u) o[16 * u + lr] = __builtin_fmaf(accl[u][r], kLoUnscale, acc[u][r]) * inv;
  }
}

// Y[m][j] = silu(G[m][2j]) * G[m][2j+1] (gate/up rows interleaved)
__global__ void __launch_bounds__(kRowThreads) swiglu(float* Y, int ldy, const float* Gb, int ldg, int F) {
  const int m = blockIdx.x;
  const float* g = Gb + (uint64_t)m * ldg;
  for (int j = threadIdx.x; j < F; j += blockDim.x) {
    const float y0 = g[2 * j], y1 = g[2 * j + 1];
    Y[(uint64_t)m * ldy + j] = y0 / (1.0f + expf(-y0)) * y1;
  }
}

// R = A + B elementwise (the lane block's residual update R_l = R_{l-1} + P_l)
__global__ void __launch_bounds__(256) radd(float* R, const float* A, const float* B, uint64_t n) {
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x)
    R[i] = A[i] + B[i];
}

}  // namespace pf
}  // namespace kie

using namespace kie;

// Scratch of kie_prefill_batched_noalloc: one array per GPU, part of the
// library's code object, so that callers that cannot allocate device memory
// (HIP graph capture, tight serving loops) can still run the batched
// prefill.  Its host-side name is not a device address: host code uses the
// pointer kie_internal_noalloc_scratch() obtains for the current device.
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

// The device address of `scratch` on `device` (which must be the current
// device), looked up once per device and kept.  Thread-safe.
extern "C" hipError_t kie_internal_noalloc_scratch(int device, void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices || !ptr) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[device] = p;
  }
  *ptr = addr[device];
  return hipSuccess;
}

static hipError_t launch_gemm(bool add, float* Out, int ldo, const float* A, int lda, const uint16_t* Wm, int M, int N,
                              int K, int32_t* state, hipStream_t st) {
  const dim3 grid((N + pf::BN - 1) / pf::BN, (M + pf::BM - 1) / pf::BM);
  if (add) {
    hipLaunchKernelGGL(pf::gemm16<true>, grid, dim3(256), 0, st, Out, ldo, A, lda, Wm, M, N, K, state);
  } else {
    hipLaunchKernelGGL(pf::gemm16<false>, grid, dim3(256), 0, st, Out, ldo, A, lda, Wm, M, N, K, state);
  }
  return hipGetLastError();
}

// every layer of one chunk of prompt tokens; asynchronous on `st`
static void launch_attention(const Dims& m, int l, float* Ao, const float* Qn, uint16_t* kv, int pos0, int C,
                             hipStream_t st) {
  const dim3 fa_grid((C + pf::FQ - 1) / pf::FQ, m.H);
  switch (m.hd) {
    case 32: hipLaunchKernelGGL(pf::attention_mfma<32>, fa_grid, dim3(256), 0, st, Ao, Qn, kv, m, l, pos0, C); break;
    case 64: hipLaunchKernelGGL(pf::attention_mfma<64>, fa_grid, dim3(256), 0, st, Ao, Qn, kv, m, l, pos0, C); break;
    case 80: hipLaunchKernelGGL(pf::attention_mfma<80>, fa_grid, dim3(256), 0, st, Ao, Qn, kv, m, l, pos0, C); break;
    case 96: hipLaunchKernelGGL(pf::attention_mfma<96>, fa_grid, dim3(256), 0, st, Ao, Qn, kv, m, l, pos0, C); break;
    case 128: hipLaunchKernelGGL(pf::attention_mfma<128>, fa_grid, dim3(256), 0, st, Ao, Qn, kv, m, l, pos0, C); break;
    default:
      hipLaunchKernelGGL(pf::attention, dim3((C * m.H + 3) / 4), dim3(256), (size_t)4 * m.hd * sizeof(float), st, Ao,
                         Qn, kv, m, l, pos0, C);
  }
}

// every layer of one chunk of prompt tokens; asynchronous on `st`.
// Sequential block: x_{l+1} = x_l + attn + mlp, both added into X.  Lane
// block (parallel, delay d): attn_l and mlp_l both read x_l, their sum P_l
// joins the residual d layers later, x_l = R_{l-d-1} with R_l = R_{l-1} + P_l
// and R_j = x_0 for j < 0 (the decode kernel's order of additions).
extern "C" hipError_t kie_internal_prefill_chunk(const PrefillArgs* a, hipStream_t st) {
  const Dims& m = a->m;
  const int C = a->C;
  if (C <= 0) return hipSuccess;
  if (m.hd > 64 * pf::kMaxDims || (m.hd & 7)) return hipErrorInvalidValue;
  const int d = m.d, qd = m.H * m.hd, kvd = m.Hkv * m.hd, F = m.F;
  const int ly = pf_ycols(m), lg = pf_gcols(m);
  const uint64_t Cd = (uint64_t)C * d;
  float* X = a->scratch;
  float* Y = X + Cd;
  float* Gb = Y + (uint64_t)C * ly;
  float* Qn = Gb + (uint64_t)C * lg;
  float* Ao = Qn + (uint64_t)C * qd;
  float* Pp = Ao + (uint64_t)C * qd;  // lane block: P [C][d], then R [delay + 2][C][d]
  float* R = Pp + Cd;
  const int nslot = m.delay + 2;
  auto Rslot = [&](int j) -> float* { return j < 0 ? X : R + (uint64_t)(j % nslot) * Cd; };
  hipError_t e;
  hipLaunchKernelGGL(pf::embed, dim3(C), dim3(pf::kRowThreads), 0, st, X, a->W, a->pl.embed, a->tokens, d, m.V,
                     a->state);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  for (int l = 0; l < m.L; ++l) {
    const uint16_t* Wl = a->W + (uint64_t)l * a->pl.layer_stride;
    const float* xin = m.parallel ? Rslot(l - m.delay - 1) : X;
    hipLaunchKernelGGL(pf::rmsnorm, dim3(C), dim3(pf::kRowThreads), 0, st, Y, ly, xin, d, Wl + a->pl.attn_norm, m.eps);
    if ((e = launch_gemm(false, Gb, lg, Y, ly, Wl + a->pl.wqkv, C, qd + 2 * kvd, d, a->state, st)) != hipSuccess) return e;
    hipLaunchKernelGGL(pf::rope_kv, dim3(C), dim3(pf::kRowThreads), 0, st, Qn, Gb, lg, a->kv, a->rope, m, l, a->pos0);
    launch_attention(m, l, Ao, Qn, a->kv, a->pos0, C, st);
    if (m.parallel) {
      // P = attn; P += mlp; R_l = R_{l-1} + P
      if ((e = launch_gemm(false, Pp, d, Ao, qd, Wl + a->pl.wo, C, d, qd, a->state, st)) != hipSuccess) return e;
    } else {
      if ((e = launch_gemm(true, X, d, Ao, qd, Wl + a->pl.wo, C, d, qd, a->state, st)) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(pf::rmsnorm, dim3(C), dim3(pf::kRowThreads), 0, st, Y, ly, xin, d, Wl + a->pl.mlp_norm, m.eps);
    if ((e = launch_gemm(false, Gb, lg, Y, ly, Wl + a->pl.wgu, C, 2 * F, d, a->state, st)) != hipSuccess) return e;
    hipLaunchKernelGGL(pf::swiglu, dim3(C), dim3(pf::kRowThreads), 0, st, Y, ly, Gb, lg, F);
    if (m.parallel) {
      if ((e = launch_gemm(true, Pp, d, Y, ly, Wl + a->pl.wd, C, d, F, a->state, st)) != hipSuccess) return e;
      const int blocks = (int)((Cd + 255) / 256 < 4096 ? (Cd + 255) / 256 : 4096);
      hipLaunchKernelGGL(pf::radd, dim3(blocks), dim3(256), 0, st, Rslot(l), Rslot(l - 1), Pp, Cd);
    } else {
      if ((e = launch_gemm(true, X, d, Y, ly, Wl + a->pl.wd, C, d, F, a->state, st)) != hipSuccess) return e;
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}
