/*
 * zaya.h — C ABI of the ZAYA1 decoder-block forward on AMD Instinct MI355X (gfx950).
 *
 * The operation is the ZAYA1 decoder layer as the nnterp encyclopedia page for
 * nnterp.families.zaya ("ZAYA1") describes it:
 *   h   = merge_a(self_attn(input_layernorm(x)), x)            ("The Notes / The block, in order")
 *   out = merge_m(mlp(post_attention_layernorm(h)), h)
 *   merge(o, r) = (o + hidden_states_bias) * hidden_states_scale + (r + residual_bias) * residual_scale
 * with compressed convolutional attention ("Queries and keys are convolved, normed to
 * √head_dim and the keys scaled"), grouped-query attention, and a top-1 mixture of
 * SwiGLU experts beside a skip class whose router state carries from block to block
 * ("One expert per token, chosen beside a skip class"). The stream is float32; every
 * other tensor is in the load dtype ("The stream is float32 whatever the load").
 * The decode state per attention layer is the KV cache plus conv_state [B, C, 2] and
 * prev_hs [B, H] (JANGTQ2 model card, "Architecture Summary").
 *
 * Conventions for every entry point:
 *  - Pointers named *_dev or documented as device point to device memory of the
 *    current HIP device; host pointers are documented as such.
 *  - All memory is owned by the caller. The library allocates nothing, keeps no
 *    global state (apart from the per-thread benchmark hook zaya_set_stage_events)
 *    and is re-entrant; each call enqueues work on `stream` (a
 *    hipStream_t passed as void*; NULL = the null stream) and returns without
 *    waiting for it.
 *  - Every check happens on the host before the first launch: on any error nothing
 *    is enqueued and no output is written. The return value is ZAYA_OK (0) or one of
 *    the negative ZAYA_E* codes; zaya_last_error() gives the message of the calling
 *    thread's last failure.
 *  - Layouts are dense, row-major, innermost dimension last.
 *  - act = the load dtype of the configuration (ZAYA_BF16 or ZAYA_F32).
 */
#ifndef ZAYA_H_
#define ZAYA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZAYA_ABI_VERSION 4

enum zaya_dtype { ZAYA_F32 = 0, ZAYA_BF16 = 1 };

/* Storage of the expert weights W_gu and W_dn. ZAYA_EXPERTS_ACT: the act dtype, like
 * every other weight. ZAYA_EXPERTS_FP8_E4M3: one byte per weight in the OCP FP8 E4M3
 * format (sign, 4 exponent bits with bias 7, 3 mantissa bits; finite values only), with
 * one fp32 scale per weight row: the weight is code_value * scale. A low-precision
 * deployment of the experts, like the quantized ZAYA1 bundles (the JANGTQ2 card's
 * "Quantization" section); it needs act_dtype ZAYA_BF16. */
/* ZAYA_EXPERTS_ACT_PACKED, ZAYA_EXPERTS_FP8_E4M3_PACKED: as ZAYA_EXPERTS_ACT and
 * ZAYA_EXPERTS_FP8_E4M3, with W_gu and W_dn in the packed layouts that zaya_pack_experts
 * writes (see there); the arithmetic is the same bit for bit, only the order of the weight
 * bytes in memory differs (the FP8 row scales keep their layout). */
enum zaya_expert_format {
  ZAYA_EXPERTS_ACT = 0,
  ZAYA_EXPERTS_FP8_E4M3 = 1,
  ZAYA_EXPERTS_ACT_PACKED = 2,
  ZAYA_EXPERTS_FP8_E4M3_PACKED = 3
};

enum zaya_status {
  ZAYA_OK = 0,
  ZAYA_EINVAL = -1,     /* a required pointer is NULL, or B/S <= 0 */
  ZAYA_ESHAPE = -2,     /* configuration outside what the kernels support */
  ZAYA_EDTYPE = -3,     /* unknown act dtype or expert format, or an unsupported pairing */
  ZAYA_EWORKSPACE = -4, /* workspace NULL or smaller than the *_workspace_bytes query */
  ZAYA_ECACHE = -5,     /* cache_len[b] < 0 or cache_len[b] + S > cap */
  ZAYA_EALIAS = -6,     /* an output aliases an input it must not alias */
  ZAYA_EHIP = -7        /* a HIP launch failed */
};

/* Block shape ("Config" and "Printout" on the nnterp page). Supported: head_dim in
 * {64, 128}; n_heads % n_kv_heads == 0 with n_heads / n_kv_heads in {1, 2, 4, 8};
 * rope_dim even and <= head_dim; conv_k 3 or 2 (with conv_k 2 in fp32, head_dim 64 or
 * n_heads / n_kv_heads <= 4); n_experts + 1 <= 32; hidden a multiple of 256 and <= 4096;
 * expert_inter a multiple of 64; router_hidden == 256. */
typedef struct zaya_block_config {
  int hidden;          /* H (hidden_size) */
  int n_heads;         /* query heads (num_attention_heads) */
  int n_kv_heads;      /* key/value heads (num_key_value_heads) */
  int head_dim;        /* d */
  int rope_dim;        /* rotated leading dims of each head (partial_rotary_factor * d) */
  float rope_theta;    /* rotary base */
  int conv_k;          /* q/k convolution: 3 = one depthwise kernel-3 conv; 2 = depthwise
                          kernel 2 then grouped kernel 2, one group per head ("Printout") */
  int n_experts;       /* E routed experts; the router scores E + 1 classes (last = skip) */
  int expert_inter;    /* I (moe_intermediate_size) */
  int router_hidden;   /* R (router down_proj width) */
  int sliding_window;  /* < 0: off; else key k visible from query q iff 0 <= p_q - p_k <= window */
  float rms_eps;       /* rms_norm_eps */
  int act_dtype;       /* enum zaya_dtype */
  int expert_format;   /* enum zaya_expert_format (0: the act dtype) */
} zaya_block_config;

/* Device pointers to one block's parameters, act dtype unless noted.
 * W_qkv [n_heads*d + n_kv_heads*d + 2*(n_kv_heads*d/2), H]: rows q_proj, k_proj,
 *   v_proj_current, v_proj_delayed ("Printout": ZayaCCAProjection).
 * conv_w [C, 3], conv_b [C], C = (n_heads + n_kv_heads) * d: the q channels (head-major)
 *   then the k channels; tap 2 multiplies the current token. With conv_k == 2, conv_w
 *   is [C, 2] (conv_qk_depthwise: tap 0 the previous token, tap 1 the current) and
 *   conv2_w [C, 2, d], conv2_b [C] are conv_qk_grouped: output channel, tap (0 previous,
 *   1 current), input channel within the output channel's head; both are required then
 *   and ignored with conv_k == 3.
 * temp [n_kv_heads]: key temperature. W_o [H, n_heads*d].
 * a_* / m_* [H]: hidden_states_bias (hsb), hidden_states_scale (hss), residual_bias
 *   (rb), residual_scale (rs) of the attention and MoE merges.
 * r_Wd [R, H], r_bd [R], r_rss [R] (router_states_scale), r_norm_g [R], r_W1, r_W2
 *   [R, R], r_b1, r_b2 [R], r_Wout [E+1, R].
 * bal_bias: fp32 [E+1] (balancing_biases). W_gu [E, 2I, H]: gate rows then up rows.
 * W_dn [E, H, I]. With expert_format ZAYA_EXPERTS_FP8_E4M3, W_gu and W_dn hold E4M3
 * bytes in the same layouts and W_gu_scale fp32 [E, 2I], W_dn_scale fp32 [E, H] their
 * row scales (both required); with ZAYA_EXPERTS_ACT the two scale pointers are
 * ignored. */
typedef struct zaya_block_weights {
  const void* ln1_g;
  const void* W_qkv;
  const void* conv_w;
  const void* conv_b;
  const void* temp;
  const void* W_o;
  const void* a_hsb;
  const void* a_hss;
  const void* a_rb;
  const void* a_rs;
  const void* ln2_g;
  const void* r_Wd;
  const void* r_bd;
  const void* r_rss;
  const void* r_norm_g;
  const void* r_W1;
  const void* r_b1;
  const void* r_W2;
  const void* r_b2;
  const void* r_Wout;
  const float* bal_bias;
  const void* W_gu;
  const void* W_dn;
  const void* m_hsb;
  const void* m_hss;
  const void* m_rb;
  const void* m_rs;
  const float* W_gu_scale;
  const float* W_dn_scale;
  const void* conv2_w;
  const void* conv2_b;
} zaya_block_weights;

/* Per-block decode state (JANGTQ2 card, "Architecture Summary"): the KV cache plus
 * conv_state and prev_hs. K, V [B, n_kv_heads, cap, d]; new tokens are written at
 * positions cache_len[b] .. cache_len[b]+S-1. conv_state [B, C, 2]: with conv_k == 3
 * slot 0 = the q/k conv input two tokens back, slot 1 = one token back; with conv_k
 * == 2 slot 0 = the input one token back, slot 1 = the depthwise conv's output one
 * token back. prev_hs [B, H]: the
 * previous token's normed input (attention_norm_output). A sequence with
 * cache_len[b] == 0 is fresh: its history reads as zeros whatever the buffers hold.
 * conv_state and prev_hs are updated in place; cache_len is never written (the
 * caller advances it). cache_len is a host array (required); cache_len_dev is an
 * optional device copy of the same values (if NULL the library stages a copy in the
 * workspace with an asynchronous host-to-device copy).
 * ring != 0 makes K and V a ring buffer for a sliding-window block (the 74B preview's
 * hybrid_sliding blocks, "Queries and keys are convolved ..." on the nnterp page): the
 * token at position p lives in slot p % cap, so a window of W needs only cap = W + 1
 * slots whatever the sequence length. It needs sliding_window >= 0 and cap >=
 * sliding_window + 1; cache_len may then exceed cap. A prefill (S > 1) into a ring
 * needs fresh sequences (every cache_len[b] == 0): the chunk's keys are formed in the
 * workspace and the last min(S, cap) positions stored.
 * Host and device lengths: validation and a few launch sizes come from the host array,
 * the kernels read cache_len_dev. A call captured in a HIP graph and replayed after the
 * caller advanced cache_len_dev (not the host array, which a graph cannot see) is
 * valid for zaya_block_decode as long as every device length stays below cap (linear
 * cache; a ring has no limit): the decode attention derives each sequence's key chunks
 * from its device length and the step always forms the delayed value. A position at or
 * past cap of a linear cache is never written (nor read), so exceeding it drops keys
 * instead of faulting. zaya_block_prefill takes its attention split from the host
 * lengths: a captured prefill is valid only for the lengths it was captured with. */
typedef struct zaya_cca_cache {
  void* K;
  void* V;
  int cap;
  void* conv_state;
  void* prev_hs;
  const int32_t* cache_len;
  const int32_t* cache_len_dev;
  int ring;
} zaya_cca_cache;

/* Optional debug taps, named after "The API / support()" on the nnterp page. Each
 * non-NULL pointer (device) receives a copy; NULL taps cost nothing.
 * T = B*S rows; layouts:
 *   attention_norm_output, mlp_norm_output [B,S,H] act; attention_queries [B,nh,S,d];
 *   attention_keys, attention_values [B,nkv,S,d]; attention_premix [B,S,nh*d];
 *   attention_output [B,S,H] act; layer_mid [B,S,H] fp32; router_logits [B,S,E+1] act;
 *   expert_classes [B,S] int32 (E = skip); expert_indices [B,S] int32;
 *   expert_weights [B,S] act; bucket_offsets [E+1] int32; bucket_ids [T] int32 (first
 *   bucket_offsets[E] used); mlp_neurons [T, I] act in bucket order; routed_output,
 *   mlp_output [B,S,H] act; layer_output [B,S,H] fp32; router_state [B,S,R] act. */
typedef struct zaya_taps {
  void* attention_norm_output;
  void* attention_queries;
  void* attention_keys;
  void* attention_values;
  void* attention_premix;
  void* attention_output;
  float* layer_mid;
  void* mlp_norm_output;
  void* router_logits;
  int32_t* expert_classes;
  int32_t* expert_indices;
  void* expert_weights;
  int32_t* bucket_offsets;
  int32_t* bucket_ids;
  void* mlp_neurons;
  void* routed_output;
  void* mlp_output;
  float* layer_output;  /* [B,S,H] fp32: the stream leaving the block (same as x_out) */
  void* router_state;   /* [B,S,R] act: the router state handed to the next block */
} zaya_taps;

/* Workspace (device bytes) needed by one block call of B sequences of S tokens
 * (decode != 0: the zaya_block_decode path, S must be 1). Returns 0 for an invalid
 * configuration. The workspace needs 256-byte alignment. */
size_t zaya_block_workspace_bytes(const zaya_block_config* cfg, int B, int S, int decode);

/* One block forward over B sequences of S new tokens.
 * x [B,S,H] fp32 (device; must not alias x_out). router_state_in [B,S,R] act: the
 * previous block's router state (NULL = block-0 semantics: no state is added).
 * x_out [B,S,H] fp32: layer_output. router_state_out [B,S,R] act: the state handed
 * to the next block (may not alias router_state_in). cache: the decode state; may be
 * NULL for fresh sequences (then keys and values live in the workspace).
 * taps: NULL or debug outputs. */
int zaya_block_prefill(const zaya_block_config* cfg, const zaya_block_weights* w, int B, int S,
                       const float* x, const void* router_state_in, float* x_out, void* router_state_out,
                       const zaya_cca_cache* cache, const zaya_taps* taps, void* workspace,
                       size_t workspace_bytes, void* stream);

/* One decode step: one new token per sequence (S = 1). x [B,H] fp32;
 * router_state_in/out [B,R]; cache required. Same contract as zaya_block_prefill. */
int zaya_block_decode(const zaya_block_config* cfg, const zaya_block_weights* w, int B, const float* x,
                      const void* router_state_in, float* x_out, void* router_state_out,
                      const zaya_cca_cache* cache, const zaya_taps* taps, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Allocation-free decode step, for callers that cannot allocate device memory or hand
 * the library a workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. Same arguments and contract as zaya_block_decode without the
 * workspace: the intermediates live in a static device array of
 * ZAYA_NOALLOC_SCRATCH_BYTES bytes (64 MiB: a decode step of 64 sequences at the
 * ZAYA1-8B widths needs about 43 MiB) that each device the library runs on holds from
 * the first call on it until the process ends. Call with the stream's device current.
 * Returns ZAYA_EWORKSPACE, with nothing launched, when the step needs more than the
 * array (zaya_block_workspace_bytes(cfg, B, 1, 1) > ZAYA_NOALLOC_SCRATCH_BYTES), and
 * ZAYA_EHIP if the array's device address cannot be obtained. Makes no hipMalloc,
 * hipFree or other allocating call. Every call on one device shares that device's array,
 * which keeps the last call's contents (no kernel reads a byte of it before writing it
 * in the same call, so nothing needs clearing): calls that overlap on one device (two
 * streams, or two threads) race, and the caller must serialise them. Under graph
 * capture pass cache_len_dev, so no host-to-device copy of the lengths is recorded. */
#define ZAYA_NOALLOC_SCRATCH_BYTES 67108864
int zaya_block_decode_noalloc(const zaya_block_config* cfg, const zaya_block_weights* w, int B, const float* x,
                              const void* router_state_in, float* x_out, void* router_state_out,
                              const zaya_cca_cache* cache, const zaya_taps* taps, void* stream);

/* Stack: embedding (tied with lm_head), n_layers blocks, final norm, lm_head
 * ("The block": embed_tokens -> layers x 40 -> norm -> lm_head; "The stream is float32
 * whatever the load": the embedding is shifted and scaled, then cast to fp32;
 * "The readout and the tokenizer": no cap or scale on the logits). */
typedef struct zaya_stack_config {
  zaya_block_config block;
  int n_layers;
  int vocab;  /* a multiple of 4 (the head stores four logits per lane), else ZAYA_ESHAPE */
  /* Which blocks use block.sliding_window (the 74B preview's hybrid_sliding blocks are
   * every other block, same page and section as the ring above): 0 = all of them; 1 =
   * blocks 0, 2, 4, ... (the others attend to the whole prefix); 2 = blocks 1, 3, 5, ... */
  int window_layers;
} zaya_stack_config;

/* embed [vocab, H] act (also the lm_head weight), emb_shift [H], emb_scale [H],
 * final_g [H]; blocks: host array of n_layers weight structs (device pointers). */
typedef struct zaya_stack_weights {
  const void* embed;
  const void* emb_shift;
  const void* emb_scale;
  const void* final_g;
  const zaya_block_weights* blocks;
} zaya_stack_weights;

size_t zaya_stack_workspace_bytes(const zaya_stack_config* cfg, int B, int S);

/* ids [B,S] int32 device, each in [0, vocab) (ids outside read row 0 — never out of
 * bounds); logits [B,S,vocab] act device. caches: NULL, or a host array of n_layers
 * cache structs. taps: NULL or a host array of n_layers tap structs. */
int zaya_stack_forward(const zaya_stack_config* cfg, const zaya_stack_weights* w, int B, int S,
                       const int32_t* ids, void* logits, const zaya_cca_cache* caches, const zaya_taps* taps,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Expert weights in the packed layout (weight preparation, done once per block; the
 * experts are the "Printout"'s ZayaExperts, stacked as the JANGTQ2 card's "Expert layout"
 * table describes). A grouped expert GEMM streams 128 weight rows at a time, 128 bytes of
 * K per row per step; row-major, each step touches 128 rows a row length apart. Packed,
 * the rows come in groups of 128 and each group stores its 128-byte K slices one after
 * another (slice s of every row of the group, rows in order, then slice s + 1), so a
 * group is one contiguous run. W_gu [E, 2I, H]: group j of expert e holds 16-row blocks
 * alternating gate rows 64 j + 16 b .. + 15 and up rows I + 64 j + 16 b .. + 15
 * (b = 0..3). W_dn [E, H, I]: group g holds rows 128 g .. 128 g + 127.
 * FP8 experts (E4M3 codes, one byte each) are packed for their own kernel, which streams
 * 16 rows of 64 bytes per step: rows in blocks of 16 (the matrix's own row order), each
 * block stored step after step (bytes 64 s .. 64 s + 63 of its 16 rows, row after row),
 * so a step is one contiguous KiB.
 * cfg: the block configuration; its expert_format says the element type (act dtype:
 * ZAYA_EXPERTS_ACT or _ACT_PACKED; FP8: ZAYA_EXPERTS_FP8_E4M3 or _FP8_E4M3_PACKED). W_gu,
 * W_dn: row-major device inputs as in zaya_block_weights. W_gu_packed, W_dn_packed: device
 * outputs of the same byte sizes, caller-owned, overlapping neither input nor each other
 * (ZAYA_EALIAS). Enqueued on stream, asynchronous; the inputs may be freed once the stream
 * has passed the copy. Blocks then run with expert_format ZAYA_EXPERTS_ACT_PACKED or
 * ZAYA_EXPERTS_FP8_E4M3_PACKED and the packed pointers as W_gu / W_dn (FP8: the same row
 * scales). */
int zaya_pack_experts(const zaya_block_config* cfg, const void* W_gu, const void* W_dn, void* W_gu_packed,
                      void* W_dn_packed, void* stream);

/* Benchmark instrumentation (not needed for correct use). The block forward runs as
 * ZAYA_N_STAGES stages in this order: input norm, q/k/v projection, CCA projection,
 * attention, o_proj + merge, post-attention norm, router down_proj, router MLP +
 * selection, buckets, expert gate/up, expert down + merge. events: host array of
 * ZAYA_N_STAGES + 1 hipEvent_t handles (passed as void*) created by the caller. While
 * set (per calling thread), each zaya_block_prefill / zaya_block_decode records
 * events[k] on its stream right before stage k and events[ZAYA_N_STAGES] after the
 * last one, so hipEventElapsedTime(events[k], events[k+1]) is stage k's duration.
 * n == 0 or events == NULL switches recording off. Returns ZAYA_EINVAL if n is neither
 * 0 nor ZAYA_N_STAGES + 1. The array is copied; the events must outlive the calls. */
#define ZAYA_N_STAGES 11
int zaya_set_stage_events(void* const* events, int n);
/* Name of stage k (0 <= k < ZAYA_N_STAGES), or "" out of range. */
const char* zaya_stage_name(int k);

/* Benchmark probe of the matrix cores (not needed for correct use): enqueues n_wg
 * workgroups of 256 threads on `stream`; each wave runs `iters` rounds of eight
 * independent 32x32x16 bf16 MFMAs on register operands (no memory traffic in the
 * loop) and writes one float per thread to sink[0 .. 256 n_wg) (device memory, owned by
 * the caller). *flops (host pointer, may be NULL) receives the dense flops the launch
 * performs, so flops / elapsed time is the attainable bf16 MFMA rate. Returns
 * ZAYA_EINVAL if n_wg <= 0, iters <= 0 or sink is NULL, ZAYA_EHIP if the launch fails. */
int zaya_probe_mfma_bf16(int n_wg, int iters, float* sink, void* stream, double* flops);

/* Benchmark probe of HBM reads (not needed for correct use): enqueues n_wg workgroups
 * of 256 threads on `stream` that read every byte of src[0 .. bytes) (device memory,
 * 16-byte aligned, bytes a multiple of 16) once with non-temporal 16-byte loads and
 * write one float per thread to sink[0 .. 256 n_wg) (device memory). bytes / elapsed
 * time is the attainable read rate. Returns ZAYA_EINVAL on a NULL pointer, n_wg <= 0,
 * or a misaligned or short buffer, ZAYA_EHIP if the launch fails. */
int zaya_probe_hbm_read(const void* src, size_t bytes, int n_wg, float* sink, void* stream);

/* Message of the calling thread's last failed call ("" if none). */
const char* zaya_last_error(void);
/* Name of a status code. */
const char* zaya_status_str(int status);
/* ZAYA_ABI_VERSION of the built library. */
int zaya_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ZAYA_H_ */
