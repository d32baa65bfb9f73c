/*
 * kie.h - C ABI of the MI355X batch-1 fp16 decode monokernel.
 *
 * Pages cited (by title; the shorthand used below in brackets):
 *   [Malay explainer] "Startup Perancis Ini Kata Perisian Sahaja Cukup untuk
 *     Pecutkan LLM 30x Lebih Pantas pada GPU Sedia Ada": approach list
 *     ("Monokernel", "Delayed Tensor Parallelism (DTP)", lane-structured
 *     transformer bullets), results table "Laneformer 2B: Keputusan yang
 *     Ditunjukkan";
 *   [Vietnamese explainer] "Kog: 'Phần mềm hóa rồng' - Tăng tốc suy luận AI
 *     gấp 30 lần mà không cần phần cứng mới": the same list and table;
 *   [Czech explainer] "Startup Kog dosahuje 3 000 tokenů/s na běžných GPU –
 *     software poráží custom čipy": section "Software versus křemík";
 *   [Chinese feature] the lynxflow.co article on Kog's low-level GPU tuning
 *     (its first heading: "一场围绕“现有GPU”的推理竞赛"), section
 *     "需求变化迫使Kog“做大”" on memory capacity and bandwidth.
 *
 * What is computed.  Single-request (batch 1) greedy decoding of a
 * decoder-only transformer with fp16 weights, run as ONE persistent GPU
 * kernel per call: prefill, every decode step, the LM head and the greedy
 * argmax all run inside the kernel without host round trips between layers
 * or tokens.  This is the problem the Kog Inference Engine pages state
 * (explainer pages, "Monokernel" bullet of the approach list and the
 * results table: FP16, batch size 1, no quantization, no speculative
 * decoding, no pruning, tokens per second per request; Czech explainer,
 * "Software versus křemík" section: one persistent program running prefill,
 * decode and LM-head sampling in one go, without per-launch overhead or grid
 * synchronisations).  The pages do not define the block; this library
 * implements the Llama-style pre-norm block (RMSNorm, rotate-half RoPE,
 * causal softmax attention with 1/sqrt(head_dim) scale, SwiGLU, untied
 * embedding and LM head), and the lane-structured parallel block whose
 * residual update is delayed by `lane_delay` layers (the pages' Laneformer
 * lanes with Delayed Tensor Parallelism, delta = 2).
 *
 * Numerics: fp16 weights and KV cache; fp32 activations, residual stream and
 * accumulation; RoPE angles from a table computed in double precision;
 * greedy argmax takes the lowest token id among equal maxima.
 *
 * Memory.  The caller owns every device buffer (allocate with any allocator,
 * e.g. PyTorch) and keeps it alive while the context uses it; the library
 * never frees caller memory.  Sizes come from kie_query_sizes().  Host
 * pointers are read only during the call that receives them.
 *
 * Streams.  `stream` arguments are hipStream_t values passed as void*.
 * Calls are asynchronous on that stream unless stated otherwise; results
 * are ready after the stream is synchronised.  A context is used by one
 * thread and one stream at a time.
 *
 * Errors.  Every call returns a kie_status; no exception crosses the ABI.
 * Argument errors are detected on the host before anything is launched.
 * Errors raised inside the kernel (a bounded wait that timed out, a token
 * id out of range) are latched in device memory and reported by
 * kie_sync_status().  kie_last_error() returns a message for the last
 * failing call on a context.
 */
#ifndef KIE_H
#define KIE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kie_status {
  KIE_OK = 0,
  KIE_ERR_INVALID_ARG = -1, /* bad pointer, size or configuration */
  KIE_ERR_HIP = -2,         /* a HIP runtime call failed */
  KIE_ERR_CAPACITY = -3,    /* position + tokens would exceed max_ctx */
  KIE_ERR_STATE = -4,       /* memory not bound / weights not loaded / no device */
  KIE_ERR_TIMEOUT = -5,     /* a wait inside the kernel exceeded the timeout */
  KIE_ERR_UNSUPPORTED = -6, /* valid model that this kernel build cannot run */
  KIE_ERR_BAD_TOKEN = -7,   /* a token id outside [0, vocab) reached the kernel */
  KIE_ERR_RANGE = -8        /* kie_prefill_batched met an activation outside the fp16 range */
} kie_status;

/* Model shape.  Rules (KIE_ERR_INVALID_ARG otherwise): all sizes > 0;
 * n_heads % n_kv_heads == 0; head_dim even and a multiple of 8;
 * d_model, n_heads*head_dim and ffn_dim multiples of 8; n_lanes divides
 * n_heads and ffn_dim; parallel_block in {0,1}; lane_delay >= 0 and 0 when
 * parallel_block == 0; max_ctx >= 1.  Shapes the kernel cannot hold in LDS
 * (or a query-group size other than 1, 2, 4) give KIE_ERR_UNSUPPORTED. */
typedef struct kie_model_config {
  int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim, ffn_dim, vocab;
  float rms_eps;      /* added to mean(x^2) inside the square root */
  double rope_base;   /* theta_i = pos * rope_base^(-2i/head_dim) */
  int32_t n_lanes;    /* lanes of the parallel block (1 = none) */
  int32_t lane_delay; /* layers between a layer and the use of its partial */
  int32_t parallel_block; /* 0: sequential pre-norm block; 1: parallel block */
  int32_t max_ctx;    /* KV-cache capacity in positions */
} kie_model_config;

/* Host-side fp16 weights (IEEE binary16 bit patterns), row-major
 * [out][in] as a Linear layer stores them.  Per-layer members point to
 * arrays of n_layers pointers.  Shapes: embed, lm_head [vocab][d_model];
 * final_norm, attn_norm[l], mlp_norm[l] [d_model]; wq[l] [n_heads*hd][d];
 * wk[l], wv[l] [n_kv_heads*hd][d]; wo[l] [d][n_heads*hd];
 * w_gate[l], w_up[l] [ffn][d]; w_down[l] [d][ffn]. */
typedef struct kie_weights {
  const uint16_t* embed;
  const uint16_t* lm_head;
  const uint16_t* final_norm;
  const uint16_t* const* attn_norm;
  const uint16_t* const* wq;
  const uint16_t* const* wk;
  const uint16_t* const* wv;
  const uint16_t* const* wo;
  const uint16_t* const* mlp_norm;
  const uint16_t* const* w_gate;
  const uint16_t* const* w_up;
  const uint16_t* const* w_down;
} kie_weights;

typedef struct kie_ctx kie_ctx; /* opaque host-side context */

/* Create a context for `cfg` on HIP device `device`.  device < 0 creates a
 * host-only context (sizes, packing and validation work; anything that needs
 * a GPU returns KIE_ERR_STATE) that assumes `256` workgroups.
 * On success *out receives the context; destroy it with kie_destroy(). */
kie_status kie_create(const kie_model_config* cfg, int device, kie_ctx** out);

/* Bytes of the three caller-owned device buffers: packed weights (every
 * parameter including the embedding table, laid out for the kernel), the
 * fp16 KV cache ([n_layers][2][n_kv_heads][max_ctx][head_dim]) and the
 * workspace (RoPE table, activation exchange words, state).  Any of the
 * output pointers may be NULL. */
kie_status kie_query_sizes(const kie_ctx* ctx, size_t* packed_weight_bytes, size_t* kv_bytes,
                           size_t* workspace_bytes);

/* Bind caller-owned device memory of at least the queried sizes (each
 * 256-byte aligned).  Initialises the workspace (RoPE table, cleared
 * exchange words) with a synchronous upload; the KV cache is not cleared.
 * Rebinding is allowed; it resets the position to 0 and unloads weights. */
kie_status kie_bind_memory(kie_ctx* ctx, void* d_packed, void* d_kv, void* d_workspace);

/* Pack the host weights into the kernel layout and upload them (blocking
 * with respect to the host: the host arrays may be freed on return).  The
 * weights stay fp16 exactly as given: the pages' results are for FP16
 * decoding with no quantization or pruning (Malay and Vietnamese explainers,
 * results table "Laneformer 2B"), and decoding at batch 1 is bound by reading
 * every weight from memory once per token (Chinese feature, section "需求变化迫使Kog“做大”", on decode being
 * memory-bandwidth bound), so the layout only reorders them for 16-byte
 * coalesced loads (row pairs in 1-KB chunks; RoPE partners and gate/up rows
 * paired) and adds nothing.  src must hold every pointer of kie_weights
 * (KIE_ERR_INVALID_ARG otherwise); KIE_ERR_STATE before kie_bind_memory;
 * KIE_ERR_HIP if an upload fails. */
kie_status kie_load_weights(kie_ctx* ctx, const kie_weights* host_src, void* stream);

/* Run the prompt d_prompt[0..n_prompt) (device int32 ids) at positions
 * pos..pos+n_prompt-1 (pos is 0 after binding), fill the KV cache and write
 * the greedy next token t1 to *d_next_token (device, may be NULL) and the
 * last position's logits [vocab] to d_logits (device fp32, may be NULL).
 * Afterwards position += n_prompt and t1 is the pending input token.  The
 * prompt runs through the same persistent decode kernel, one position per
 * step, with the LM head only at the last position: the pages' monokernel
 * covers prefill as well as decode and LM-head sampling in one persistent
 * program (Czech explainer, "Software versus křemík" section).  Long
 * prompts are split into several launches (kie_set_launch_steps).
 * KIE_ERR_INVALID_ARG for an empty prompt, KIE_ERR_CAPACITY if
 * pos + n_prompt > max_ctx, KIE_ERR_STATE if memory or weights are missing;
 * an id outside [0, vocab) latches KIE_ERR_BAD_TOKEN (kie_sync_status). */
kie_status kie_prefill(kie_ctx* ctx, const int32_t* d_prompt, int32_t n_prompt, int32_t* d_next_token,
                       float* d_logits, void* stream);

/* Bytes of device scratch kie_prefill_batched needs to process chunk_tokens
 * prompt tokens per chunk (fp32 activations of the chunk). */
kie_status kie_prefill_scratch_bytes(const kie_ctx* ctx, int32_t chunk_tokens, size_t* bytes);

/* kie_prefill with the prompt batched: the same result (KV cache rows for
 * positions pos..pos+n_prompt-1, t1, the last position's logits, position
 * += n_prompt), computed as dense products on the matrix cores.  The pages'
 * monokernel runs prefill on the GPU (Czech explainer, "Software versus
 * křemík" section); batching the prompt reads every weight once per chunk
 * of tokens instead of once per token.  All prompt tokens but the last go
 * through batched GEMMs (fp32 activations, fp16 weights, fp32 accumulation;
 * on the fp16 matrix cores, each activation a entering as hi = fp16(a) and
 * lo = fp16((a - hi) * 2^11), the two products accumulated apart and added
 * as hi + 2^-11 lo, so they keep fp32 accuracy to ~2^-22 relative for
 * 2^-14 <= |a| <= 65504 and to ~2^-25 absolute below), RoPE, fp16 KV append
 * and causal attention (likewise), chunk by chunk; the last one runs through
 * the decode kernel, which yields t1 (greedy or sampled, see
 * kie_set_sampling).  An activation above 65504 in magnitude (or not
 * finite) cannot be split: it latches KIE_ERR_RANGE (kie_sync_status).  d_scratch is caller-owned device memory (16-byte
 * aligned) of scratch_bytes; the chunk is the largest that fits, at most
 * 2048 tokens (kie_prefill_scratch_bytes gives the size for a chunk).  The
 * lane-structured block keeps its delayed residual (layer l reads
 * x_0 + P_0 + .. + P_{l-delay-1}).  ffn_dim not a multiple of 4 and a
 * one-token prompt fall back to kie_prefill.  KIE_ERR_INVALID_ARG if the
 * scratch cannot hold one token; an out-of-range id latches
 * KIE_ERR_BAD_TOKEN as in kie_prefill.  Asynchronous on `stream`. */
kie_status kie_prefill_batched(kie_ctx* ctx, const int32_t* d_prompt, int32_t n_prompt, int32_t* d_next_token,
                               float* d_logits, void* d_scratch, size_t scratch_bytes, void* stream);

/* kie_prefill_batched without a caller scratch buffer, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  The chunk activations live in a
 * fixed array of 64 MiB per GPU inside the library (held until the process
 * ends; its device address is looked up once per device by kie_create), so
 * the chunk is the largest that fits it, at most 2048 tokens.  This call
 * allocates nothing and frees nothing.  Every call on one GPU shares that
 * GPU's array and leaves its contents behind (every value is written before
 * it is read, so nothing needs clearing): calls that overlap in time on one
 * GPU, from two streams or two contexts, race and must be serialised by the
 * caller.  Result, status and errors as kie_prefill_batched;
 * KIE_ERR_UNSUPPORTED if one prompt token needs more scratch than the array
 * holds. */
kie_status kie_prefill_batched_noalloc(kie_ctx* ctx, const int32_t* d_prompt, int32_t n_prompt,
                                       int32_t* d_next_token, float* d_logits, void* stream);

/* Run n_tokens decode steps inside one persistent kernel launch per
 * kie_set_launch_steps steps: the pages' monokernel, one program for the
 * whole decode loop with no kernel launches between layers or tokens and no
 * grid synchronisations (Malay and Vietnamese explainers, "Monokernel"
 * bullet; Czech explainer, "Software versus křemík" section), emitting
 * tokens of a single request at batch 1 (results table "Laneformer 2B").
 * Step k consumes d_forced_in[k] when that
 * pointer is not NULL (teacher forcing), else the previous step's argmax (the
 * pending token for k = 0); it runs at position pos + k, writes its greedy
 * (or sampled, see kie_set_sampling) token to d_tokens_out[k] (device, may be NULL) and, when d_logits_out is not
 * NULL, its logits to d_logits_out[k*vocab .. (k+1)*vocab).  Afterwards
 * position += n_tokens and the last emitted token is pending.
 * KIE_ERR_CAPACITY if position + n_tokens > max_ctx. */
kie_status kie_decode(kie_ctx* ctx, int32_t n_tokens, int32_t* d_tokens_out, const int32_t* d_forced_in,
                      float* d_logits_out, void* stream);

/* Set the position (0 <= pos <= max_ctx) and the pending input token
 * (0 <= token < vocab) without touching the KV cache, e.g. to time the same
 * decode again.  Asynchronous on `stream`. */
kie_status kie_set_position(kie_ctx* ctx, int32_t pos, int32_t next_token, void* stream);

/* Synchronise `stream` and report errors latched by the kernel
 * (KIE_ERR_TIMEOUT, KIE_ERR_BAD_TOKEN), clearing them.  After such an error
 * the workspace's exchange state is reset (a timed-out launch can stop in the
 * middle of a step); the KV cache and the position are kept, so a caller can
 * rewind with kie_set_position and decode again. */
kie_status kie_sync_status(kie_ctx* ctx, void* stream);

/* Longest time one wait inside the kernel may take before the launch gives
 * up with KIE_ERR_TIMEOUT (default 2 000 000 us). */
kie_status kie_set_timeout_us(kie_ctx* ctx, uint64_t microseconds);

/* Stochastic LM-head sampling inside the kernel (Kog explainer, "Monokernel"
 * section: LM-head sampling runs in the persistent kernel; the sampler is
 * not named there).  For temperature T > 0 every emitted token -- the
 * prefill's t1 and each decode step's -- is the argmax over vocabulary rows i
 * of logits[i] / T + g_i, where g_i = -log(-log(u_i)) is standard Gumbel
 * noise, so the token is a draw from softmax(logits / T).  u_i = ((w >> 9) +
 * 1/2) * 2^-23 with w the first output word of Philox4x32-10 (Salmon et al.,
 * SC 2011) with key (seed mod 2^32, seed >> 32) and counter (i, position,
 * 0, 0), where position is that of the input token the logits follow from.
 * Equal scores go to the lower id.  T = 0 (the default) is greedy decoding.
 * Logits written to d_logits / d_logits_out stay unperturbed.  Applies to
 * later kie_prefill and kie_decode calls; KIE_ERR_INVALID_ARG for a negative
 * or non-finite temperature (the setting is then left unchanged). */
kie_status kie_set_sampling(kie_ctx* ctx, float temperature, uint64_t seed);

/* Debug flags.  Bit 0: one workgroup waits on a word nobody writes, which
 * must end in KIE_ERR_TIMEOUT, not a hang.  Bit 1: race-detection jitter,
 * every wave sleeps a pseudo-random 0..6 us at the start of every phase
 * (hashed from workgroup, wave, step and phase), which reorders the
 * workgroups' arrivals at every exchange; the results must stay bitwise
 * identical.  0 = normal operation. */
kie_status kie_set_debug_flags(kie_ctx* ctx, uint32_t flags);

/* Phase trace for performance analysis.  When d_trace is not NULL, the
 * first `steps` steps of every launch write, per phase and workgroup, four
 * 64-bit wall-clock stamps (phase start, input ready, stream done, phase end)
 * into device memory d_trace at index ((step*322 + phase)*n_workgroups + wg)*4
 * (phase 321 is the end-of-step exchange).  The caller owns the buffer
 * (steps*322*n_workgroups*32 bytes).  NULL / 0 turns tracing off. */
kie_status kie_set_trace(kie_ctx* ctx, void* d_trace, int32_t steps);

/* CPU-only: the phase order of one decode step for `cfg` on n_workgroups
 * workgroups (the phase index of the trace above): phase p runs kind[p] of
 * layer layer[p], kinds 0 QKV, 1 attention, 2 O, 3 gate/up, 4 down, 5 LM
 * head (layer = n_layers).  The sequential block runs each layer's phases in
 * that kind order.  The parallel block runs QKV, gate/up, attention, O, down
 * per layer; with a residual delay of two or more layers (and two or fewer
 * query heads per KV head) it is software-pipelined, layer l's attention
 * followed by layer l + 1's QKV and gate/up before layer l's O and down: the
 * delayed residual (the Laneformer lanes with Delayed Tensor Parallelism of
 * the explainer pages' approach list) makes layer l + 1's input independent
 * of layer l.  Writes 5 * n_layers + 1 entries;
 * KIE_ERR_INVALID_ARG if n is smaller or the arrays are NULL,
 * KIE_ERR_UNSUPPORTED for a shape the kernel does not run. */
kie_status kie_phase_order(const kie_model_config* cfg, int32_t n_workgroups, int32_t* kind, int32_t* layer,
                           int32_t n);

/* CPU-only: which lanes each workgroup's work belongs to.  Lane j owns the
 * query heads [j*H/n_lanes, (j+1)*H/n_lanes) (a KV head belongs to the lanes
 * of its query heads) and the FFN columns [j*F/n_lanes, (j+1)*F/n_lanes).
 * For kind k = 0 (QKV rows), 1 (attention: the workgroup's KV head), 2
 * (gate/up rows), lane_lo[k*n + w] .. lane_hi[k*n + w] are the lowest and
 * highest lane of workgroup w's work (-1 where it has none of that kind),
 * n = n_workgroups.  The kernel numbers its workgroups XCD by XCD
 * (workgroup w runs on XCD w / (n / 8)), so for a lane-structured model
 * whose lanes each fall on one block of n / n_lanes workgroups, each lane's
 * attention heads and FFN columns run on one XCD: the Laneformer lanes of
 * the pages (Malay and Vietnamese explainers, approach list,
 * lane-structured transformer and Delayed Tensor Parallelism bullets) on the
 * chip's XCDs.  The QKV rows are packed all q, then all k, then all v, so a
 * workgroup's QKV rows belong to other lanes; the O and down projections are
 * split by output rows over every workgroup and read every lane's output.
 * KIE_ERR_INVALID_ARG for bad arguments, KIE_ERR_UNSUPPORTED for a shape the
 * kernel does not run. */
kie_status kie_lane_placement(const kie_model_config* cfg, int32_t n_workgroups, int32_t* lane_lo,
                              int32_t* lane_hi);

/* CPU-only: ring slots per wave (*depth, 8 or 10) of the decode kernel build
 * that a context for `cfg` on n_workgroups workgroups launches.  Each wave
 * streams its weight chunks through a ring of one-KB LDS slots (the weights
 * stream through on-chip memory once per token, as the monokernel pages
 * describe the weight path); the deeper ring is used for the sequential block
 * when its other LDS buffers fit beside it.  The two builds are the same
 * kernel, named kie::ring8:: and kie::ring10:: in profiler output.
 * KIE_ERR_INVALID_ARG for a bad config or NULL depth, KIE_ERR_UNSUPPORTED
 * for a shape the kernel does not run. */
kie_status kie_ring_depth(const kie_model_config* cfg, int32_t n_workgroups, int32_t* depth);

/* Most decode steps one launch runs before the library starts the next one
 * (default 512); keeps each launch short. */
kie_status kie_set_launch_steps(kie_ctx* ctx, int32_t steps);

/* CPU-only: write the packed layout of `src` for `cfg` into host_dst
 * (packed_weight_bytes from kie_query_sizes of any context for cfg). */
kie_status kie_pack_weights_host(const kie_model_config* cfg, const kie_weights* src, void* host_dst);

/* Launch shape: workgroups (= compute units), threads per workgroup, LDS
 * bytes per workgroup (the same 160 KB whichever ring depth the context
 * runs: 10 one-KB slots per wave for the sequential block when its LDS plan
 * fits beside them, 8 otherwise), and the packed element offsets of layer
 * 0's fused QKV matrix and the LM head. */
kie_status kie_launch_info(const kie_ctx* ctx, int32_t* n_workgroups, int32_t* threads, int32_t* lds_bytes,
                           int64_t* qkv_offset, int64_t* lm_offset);

/* CPU-only: check the work partition the kernel derives for `cfg` on
 * n_workgroups workgroups at context length n_ctx: every GEMV row and
 * every 512-column block of it belongs to exactly one wave, every attention
 * key of every KV head to exactly one wave, every head has exactly one merging
 * workgroup and every workgroup meets at most two heads.  On failure returns
 * KIE_ERR_INVALID_ARG and writes a message into msg (msg_len bytes). */
kie_status kie_validate_schedule(const kie_model_config* cfg, int32_t n_workgroups, int32_t n_ctx, char* msg,
                                 size_t msg_len);

/* Current position (number of cached positions). */
int32_t kie_position(const kie_ctx* ctx);

const char* kie_status_string(kie_status s);
const char* kie_last_error(const kie_ctx* ctx);
void kie_destroy(kie_ctx* ctx);

#ifdef __cplusplus
}
#endif
#endif /* KIE_H */
