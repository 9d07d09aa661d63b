// Host side of the C ABI declared in include/zaya.h: validation, workspace layout and
// launch sequencing. No device call is made before every check has passed.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <mutex>
#include <type_traits>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/zaya.h"
#include "kernels.h"

using namespace zaya;

namespace {

thread_local std::string g_err;
thread_local std::vector<hipEvent_t> g_stage_events;  // empty: no stage recording

const char* const kStageNames[ZAYA_N_STAGES] = {
    "input_norm", "qkv_proj", "cca", "attention", "o_proj_merge", "post_attn_norm",
    "router_down", "router_mlp_select", "buckets", "expert_gate_up", "expert_down_merge"};

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t act_bytes(const zaya_block_config* c) { return c->act_dtype == ZAYA_BF16 ? 2 : 4; }

bool fp8_experts(const zaya_block_config* c) {
  return c->expert_format == ZAYA_EXPERTS_FP8_E4M3 || c->expert_format == ZAYA_EXPERTS_FP8_E4M3_PACKED;
}

int check_config(const zaya_block_config* c) {
  if (!c) return fail(ZAYA_EINVAL, "config is NULL");
  if (c->act_dtype != ZAYA_BF16 && c->act_dtype != ZAYA_F32) return fail(ZAYA_EDTYPE, "act_dtype %d", c->act_dtype);
  if (c->hidden <= 0 || c->n_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 || c->n_experts <= 0 ||
      c->expert_inter <= 0 || c->router_hidden <= 0)
    return fail(ZAYA_ESHAPE, "non-positive dimension");
  if (c->head_dim != 64 && c->head_dim != 128) return fail(ZAYA_ESHAPE, "head_dim %d not in {64, 128}", c->head_dim);
  if (c->n_heads % c->n_kv_heads) return fail(ZAYA_ESHAPE, "n_heads %% n_kv_heads != 0");
  const int G = c->n_heads / c->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return fail(ZAYA_ESHAPE, "n_heads / n_kv_heads = %d not in {1,2,4,8}", G);
  if (c->rope_dim < 0 || c->rope_dim > c->head_dim || (c->rope_dim & 1))
    return fail(ZAYA_ESHAPE, "rope_dim %d must be even and <= head_dim", c->rope_dim);
  if (c->conv_k != 3 && c->conv_k != 2) return fail(ZAYA_ESHAPE, "conv_k %d not in {2, 3}", c->conv_k);
  if (c->conv_k == 2 && cca_lds_bytes(c->head_dim, G, (int)act_bytes(c), true) > 160 * 1024)
    return fail(ZAYA_ESHAPE, "conv_k 2: head_dim %d with %d query heads per key head does not fit LDS in this dtype",
                c->head_dim, G);
  if (c->n_experts + 1 > 32) return fail(ZAYA_ESHAPE, "n_experts + 1 > 32");
  if (c->hidden % 256 || c->hidden > 4096) return fail(ZAYA_ESHAPE, "hidden %d must be a multiple of 256, <= 4096", c->hidden);
  if (c->expert_inter % 64) return fail(ZAYA_ESHAPE, "expert_inter %d must be a multiple of 64", c->expert_inter);
  if (c->router_hidden != 256) return fail(ZAYA_ESHAPE, "router_hidden %d != 256", c->router_hidden);
  if (!(c->rms_eps > 0.f)) return fail(ZAYA_ESHAPE, "rms_eps must be > 0");
  if (!(c->rope_theta > 0.f)) return fail(ZAYA_ESHAPE, "rope_theta must be > 0");
  if (c->expert_format < ZAYA_EXPERTS_ACT || c->expert_format > ZAYA_EXPERTS_FP8_E4M3_PACKED)
    return fail(ZAYA_EDTYPE, "expert_format %d", c->expert_format);
  if (fp8_experts(c)) {
    if (c->act_dtype != ZAYA_BF16) return fail(ZAYA_EDTYPE, "FP8 experts need act_dtype ZAYA_BF16");
    if (c->expert_inter > 4096) return fail(ZAYA_ESHAPE, "FP8 experts: expert_inter %d > 4096", c->expert_inter);
  }
  return ZAYA_OK;
}

// Key-range chunks per query tile the prefill workspace has room for: what a call
// without cached tokens needs with the shorter of the kernels' chunk lengths, and at
// least 4 so calls after a cache can split too.
constexpr int kPrefillChunkTilesMin = 16;
int prefill_chunks_ws(const zaya_block_config* c, int S) {
  const int nc = attn_prefill_chunks(S, 0, c->sliding_window, kPrefillChunkTilesMin);
  return nc < 4 ? 4 : nc;
}

// Workspace layout of one block call.
struct Plan {
  size_t cache_len, xn, P, vdp, y2, Q, Kw, Vw, convw, prevw, O, h, hn, logits, cls, idx, wts, offsets, ids, neurons,
      part, rcnt;
  size_t gpart, gpart_bytes;  // split-K partials of the few-row GEMMs
  size_t total;
};

Plan plan_block(const zaya_block_config* c, int B, int S, int decode) {
  const size_t A = act_bytes(c);
  const size_t T = (size_t)B * S;
  const int H = c->hidden, nh = c->n_heads, nkv = c->n_kv_heads, d = c->head_dim;
  const size_t QR = (size_t)nh * d + 2 * (size_t)nkv * d;
  const int E = c->n_experts;
  const size_t C = (size_t)(nh + nkv) * d;
  Plan p{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o += align256(bytes);
    return at;
  };
  p.cache_len = take((size_t)B * 4);
  p.xn = take(T * H * A);
  p.P = take(T * QR * A);
  p.vdp = take((size_t)B * nkv * (d / 2) * A);
  p.y2 = take(c->conv_k == 2 ? T * C * A : 0);  // two-stage conv output
  p.Q = take(T * nh * d * A);
  p.Kw = take(T * nkv * d * A);  // keys/values when the caller passes no cache
  p.Vw = take(T * nkv * d * A);
  p.convw = take((size_t)B * C * 2 * A);
  p.prevw = take((size_t)B * H * A);
  p.O = take(T * nh * d * A);
  p.h = take(T * H * 4);
  p.hn = take(T * H * A);
  p.logits = take(T * (E + 1) * A);
  p.cls = take(T * 4);
  p.idx = take(T * 4);
  p.wts = take(T * A);
  p.offsets = take((size_t)(E + 1) * 4);
  p.ids = take(T * 4);
  p.rcnt = take((size_t)(E + 1) * bucket_counts_ld((int)T) * 4);
  p.neurons = take(T * c->expert_inter * A);
  p.part = decode ? take(attn_decode_part_bytes(B, nkv, nh / nkv, d))
                  : take(attn_prefill_part_bytes(B, S, nkv, nh / nkv, d, prefill_chunks_ws(c, S)));
  // split-K partials (only calls with at most 64 rows use them): 64 x max(N) x 16 parts
  const size_t maxn = std::max<size_t>(std::max<size_t>(QR, H), c->router_hidden);
  p.gpart_bytes = T <= 64 ? (size_t)64 * maxn * 16 * 4 : 0;
  p.gpart = take(p.gpart_bytes);
  p.total = o;
  return p;
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b) return false;
  const char* pa = (const char*)a;
  const char* pb = (const char*)b;
  return pa < pb + nb && pb < pa + na;
}

int check_weights(const zaya_block_config* c, const zaya_block_weights* w) {
  if (!w) return fail(ZAYA_EINVAL, "weights is NULL");
  if (fp8_experts(c) && (!w->W_gu_scale || !w->W_dn_scale))
    return fail(ZAYA_EINVAL, "FP8 experts need W_gu_scale and W_dn_scale");
  if (c->conv_k == 2 && (!w->conv2_w || !w->conv2_b))
    return fail(ZAYA_EINVAL, "conv_k 2 needs conv2_w and conv2_b");
  const void* ptrs[] = {w->ln1_g, w->W_qkv, w->conv_w, w->conv_b, w->temp, w->W_o, w->a_hsb, w->a_hss, w->a_rb,
                        w->a_rs, w->ln2_g, w->r_Wd, w->r_bd, w->r_rss, w->r_norm_g, w->r_W1, w->r_b1, w->r_W2,
                        w->r_b2, w->r_Wout, w->bal_bias, w->W_gu, w->W_dn, w->m_hsb, w->m_hss, w->m_rb, w->m_rs};
  for (size_t i = 0; i < sizeof ptrs / sizeof ptrs[0]; ++i)
    if (!ptrs[i]) return fail(ZAYA_EINVAL, "weight pointer #%zu is NULL", i);
  return ZAYA_OK;
}

#define HIPCHK(expr)                                                               \
  do {                                                                             \
    hipError_t e_ = (expr);                                                        \
    if (e_ != hipSuccess) return fail(ZAYA_EHIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

template <typename T>
int run_block(const zaya_block_config* c, const zaya_block_weights* w, int B, int S, bool decode, const float* x,
              const void* s_in, float* x_out, void* s_out, const zaya_cca_cache* cache, const zaya_taps* taps,
              char* ws, const Plan& p, int max_len, hipStream_t st) {
  // max_len: prefill, the largest cache_len + S; decode, the attention span (see launch_attn_decode)
  const int H = c->hidden, nh = c->n_heads, nkv = c->n_kv_heads, d = c->head_dim, E = c->n_experts;
  const int I = c->expert_inter, R = c->router_hidden;
  const int T_ = B * S;
  const int QR = nh * d + 2 * nkv * d;
  const int C = (nh + nkv) * d;
  const size_t A = sizeof(T);
  auto W = [](const void* q) { return static_cast<const T*>(q); };
  T* xn = (T*)(ws + p.xn);
  T* P = (T*)(ws + p.P);
  T* vdp = (T*)(ws + p.vdp);
  T* Q = (T*)(ws + p.Q);
  T* O = (T*)(ws + p.O);
  float* h = (float*)(ws + p.h);
  T* hn = (T*)(ws + p.hn);
  T* logits = (T*)(ws + p.logits);
  int32_t* cls = (int32_t*)(ws + p.cls);
  int32_t* idx = (int32_t*)(ws + p.idx);
  T* wts = (T*)(ws + p.wts);
  int32_t* offsets = (int32_t*)(ws + p.offsets);
  int32_t* ids = (int32_t*)(ws + p.ids);
  T* neurons = (T*)(ws + p.neurons);
  const zaya_taps tz{};
  const zaya_taps& tp = taps ? *taps : tz;
  auto tap_copy = [&](void* dst, const void* src, size_t bytes) -> hipError_t {
    return dst ? hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, st) : hipSuccess;
  };

  auto mark = [&](int k) -> hipError_t {
    return g_stage_events.empty() ? hipSuccess : hipEventRecord(g_stage_events[k], st);
  };

  // cache lengths on the device
  const int32_t* cl_dev;
  bool any_cached = false;
  if (cache) {
    // decode always forms the delayed value of the token before the step (the kernels
    // ignore it for fresh sequences), so a captured decode step stays valid when the
    // device-side lengths grow from zero
    any_cached = decode;
    for (int b = 0; b < B; ++b) any_cached |= cache->cache_len[b] > 0;
    if (cache->cache_len_dev) {
      cl_dev = cache->cache_len_dev;
    } else {
      HIPCHK(hipMemcpyAsync(ws + p.cache_len, cache->cache_len, (size_t)B * 4, hipMemcpyHostToDevice, st));
      cl_dev = (const int32_t*)(ws + p.cache_len);
    }
  } else {
    cl_dev = nullptr;  // the kernels read a null table as all sequences fresh
  }
  // a ring cache takes fresh prefills (checked): their keys and values are formed in the
  // workspace and the last positions stored afterwards; a decode step writes its slot
  const bool ring_prefill = cache && cache->ring && !decode;
  const int ring = cache && cache->ring && decode ? 1 : 0;
  T* Kc = cache && !ring_prefill ? (T*)cache->K : (T*)(ws + p.Kw);
  T* Vc = cache && !ring_prefill ? (T*)cache->V : (T*)(ws + p.Vw);
  const int cap = cache && !ring_prefill ? cache->cap : S;
  T* conv_state = cache ? (T*)cache->conv_state : (T*)(ws + p.convw);
  T* prev_hs = cache ? (T*)cache->prev_hs : (T*)(ws + p.prevw);

  // a1: input RMSNorm
  HIPCHK(mark(0));
  HIPCHK(launch_rmsnorm_stream<T>(x, W(w->ln1_g), xn, T_, H, c->rms_eps, st));
  HIPCHK(tap_copy(tp.attention_norm_output, xn, (size_t)T_ * H * A));
  // a2: q/k/v projections (+ the delayed value of the token before this call)
  HIPCHK(mark(1));
  float* gpart = p.gpart_bytes ? (float*)(ws + p.gpart) : nullptr;
  const T* Wvd = W(w->W_qkv) + (size_t)(nh * d + nkv * d + nkv * d / 2) * H;
  int qkv_kparts = 0;  // > 0: the CCA kernel sums the split-K partials itself
  if (decode && c->conv_k == 3 && T_ <= 64) {
    qkv_kparts = launch_gemm_pair_parts<T>(xn, H, W(w->W_qkv), H, T_, QR, prev_hs, H, Wvd, H, B, nkv * d / 2, H,
                                           gpart, p.gpart_bytes, st);
    if (qkv_kparts < 0) return fail(ZAYA_EHIP, "q/k/v split-K launch failed");
  }
  if (qkv_kparts > 0) {
    // P and vdp stay as partials
  } else if (any_cached && T_ <= 64) {  // few rows: both products share one split-K pass
    HIPCHK(launch_gemm_store_pair<T>(xn, H, W(w->W_qkv), H, T_, QR, P, QR, prev_hs, H, Wvd, H, B, nkv * d / 2, vdp,
                                     nkv * d / 2, H, gpart, p.gpart_bytes, st));
  } else {
    HIPCHK(launch_gemm_store<T>(xn, H, W(w->W_qkv), H, T_, QR, H, P, QR, gpart, p.gpart_bytes, st));
    if (any_cached)
      HIPCHK(launch_gemm_store<T>(prev_hs, H, Wvd, H, B, nkv * d / 2, H, vdp, nkv * d / 2, gpart, p.gpart_bytes, st));
  }
  // a3: convolution, residual, QK norm, temperature, rotary, value halves, state
  HIPCHK(mark(2));
  T* y2 = nullptr;
  if (c->conv_k == 2) {  // the two-stage conv first: it reads conv_state before the CCA kernel updates it
    y2 = (T*)(ws + p.y2);
    Conv2Args<T> c2{P, QR, W(w->conv_w), W(w->conv_b), W(w->conv2_w), W(w->conv2_b), conv_state, cl_dev, y2,
                    B, S, C, d};
    HIPCHK(launch_conv2<T>(c2, st));
  }
  CcaArgs<T> ca{P, QR, vdp, W(w->conv_w), W(w->conv_b), W(w->temp), conv_state, prev_hs, xn, cl_dev, Q, Kc, Vc, cap,
                (T*)tp.attention_queries, (T*)tp.attention_keys, (T*)tp.attention_values,
                B, S, H, nh, nkv, d, c->rope_dim, C, c->rope_theta, c->conv_k, y2, ring};
  if (qkv_kparts > 0) {
    ca.qkv_part = gpart;
    ca.vd_part = gpart + (size_t)T_ * QR * qkv_kparts;
    ca.kparts = qkv_kparts;
  }
  HIPCHK(launch_cca<T>(ca, st));
  if (ring_prefill) HIPCHK(launch_ring_store<T>(Kc, Vc, (T*)cache->K, (T*)cache->V, B, nkv, S, d, cache->cap, st));
  // a4: attention
  HIPCHK(mark(3));
  AttnArgs<T> aa{Q, Kc, Vc, O, cl_dev, B, S, nh, nkv, d, cap, c->sliding_window, ring};
  if (decode)
    HIPCHK(launch_attn_decode<T>(aa, (float*)(ws + p.part), max_len, st));
  else
    HIPCHK(launch_attn_prefill<T>(aa, (float*)(ws + p.part),
                                  std::min(attn_prefill_chunks(S, max_len - S, c->sliding_window,
                                                               attn_prefill_chunk_tiles((int)A, d, nh / nkv)),
                                           prefill_chunks_ws(c, S)),
                                  st));
  HIPCHK(tap_copy(tp.attention_premix, O, (size_t)T_ * nh * d * A));
  // a5: o_proj + attention merge
  HIPCHK(mark(4));
  // few rows: split-K partials, then one pass that sums them, merges and norms (a5 + a6)
  const int oparts = launch_gemm_parts<T>(O, nh * d, W(w->W_o), nh * d, T_, H, nh * d, gpart, p.gpart_bytes, st);
  if (oparts < 0) return fail(ZAYA_EHIP, "o_proj split-K launch failed");
  if (oparts > 1) {
    HIPCHK(launch_merge_norm_parts<T>(gpart, oparts, T_, H, x, W(w->a_hsb), W(w->a_hss), W(w->a_rb), W(w->a_rs), h,
                                      (T*)tp.attention_output, W(w->ln2_g), hn, c->rms_eps, st));
    HIPCHK(tap_copy(tp.layer_mid, h, (size_t)T_ * H * 4));
    HIPCHK(mark(5));
  } else {
    HIPCHK(launch_gemm_merge<T>(O, W(w->W_o), T_, H, nh * d, x, W(w->a_hsb), W(w->a_hss), W(w->a_rb), W(w->a_rs), h,
                                (T*)tp.attention_output, gpart, p.gpart_bytes, st));
    HIPCHK(tap_copy(tp.layer_mid, h, (size_t)T_ * H * 4));
    // a6: post-attention RMSNorm
    HIPCHK(mark(5));
    HIPCHK(launch_rmsnorm_stream<T>(h, W(w->ln2_g), hn, T_, H, c->rms_eps, st));
  }
  HIPCHK(tap_copy(tp.mlp_norm_output, hn, (size_t)T_ * H * A));
  // a7: router down_proj + carried state
  HIPCHK(mark(6));
  // few rows: only the split-K partials here; the router kernel sums them
  const int rparts = T_ <= 64 ? launch_gemm_parts<T>(hn, H, W(w->r_Wd), H, T_, R, H, gpart, p.gpart_bytes, st) : 0;
  if (rparts < 0) return fail(ZAYA_EHIP, "router split-K launch failed");
  if (rparts == 0)
    HIPCHK(launch_gemm_router_in<T>(hn, W(w->r_Wd), T_, R, H, W(w->r_bd), W(w->r_rss), (const T*)s_in, (T*)s_out,
                                    gpart, p.gpart_bytes, st));
  // a7/a8: router MLP, selection, skip tokens' merge
  HIPCHK(mark(7));
  RouterArgs<T> ra{(const T*)s_out, W(w->r_norm_g), W(w->r_W1), W(w->r_b1), W(w->r_W2), W(w->r_b2), W(w->r_Wout),
                   w->bal_bias, logits, cls, idx, wts, h, W(w->m_hsb), W(w->m_hss), W(w->m_rb), W(w->m_rs), x_out,
                   (T*)tp.routed_output, (T*)tp.mlp_output, T_, R, E, H, c->rms_eps};
  const bool small_buckets = T_ <= 64;
  if (!small_buckets) {
    ra.counts = (int32_t*)(ws + p.rcnt);
    ra.counts_ld = bucket_counts_ld(T_);
  }
  if (rparts > 0) {
    ra.part = gpart;
    ra.kparts = rparts;
    ra.bd = W(w->r_bd);
    ra.rss = W(w->r_rss);
    ra.s_in = (const T*)s_in;
    ra.u_out = (T*)s_out;
  }
  HIPCHK(launch_router<T>(ra, st));
  HIPCHK(tap_copy(tp.router_logits, logits, (size_t)T_ * (E + 1) * A));
  HIPCHK(tap_copy(tp.expert_classes, cls, (size_t)T_ * 4));
  HIPCHK(tap_copy(tp.expert_indices, idx, (size_t)T_ * 4));
  HIPCHK(tap_copy(tp.expert_weights, wts, (size_t)T_ * A));
  // a9: buckets (at most 64 tokens: formed by the gate/up kernel itself)
  HIPCHK(mark(8));
  if (!small_buckets) {
    HIPCHK(launch_bucket(cls, ra.counts, T_, E, offsets, ids, st));
    HIPCHK(tap_copy(tp.bucket_offsets, offsets, (size_t)(E + 1) * 4));
    HIPCHK(tap_copy(tp.bucket_ids, ids, (size_t)T_ * 4));
  }
  // a10/a11: experts, weighted combine, MoE merge
  MoeArgs<T> ma{offsets, ids, hn, W(w->W_gu), W(w->W_dn), neurons, wts, h, W(w->m_hsb), W(w->m_hss), W(w->m_rb),
                W(w->m_rs), x_out, (T*)tp.routed_output, (T*)tp.mlp_output, T_, H, I, E};
  ma.gu_scale = w->W_gu_scale;
  ma.dn_scale = w->W_dn_scale;
  ma.packed = c->expert_format == ZAYA_EXPERTS_ACT_PACKED || c->expert_format == ZAYA_EXPERTS_FP8_E4M3_PACKED;
  if (small_buckets) {
    ma.cls = cls;
    ma.offsets_out = offsets;
    ma.ids_out = ids;
  }
  const bool f8 = fp8_experts(c);  // act is bf16 (checked)
  HIPCHK(mark(9));
  if constexpr (std::is_same<T, bf16_t>::value) {
    HIPCHK(f8 ? launch_moe_gateup_f8(ma, st) : launch_moe_gateup<T>(ma, st));
  } else {
    HIPCHK(launch_moe_gateup<T>(ma, st));
  }
  if (small_buckets) {
    HIPCHK(tap_copy(tp.bucket_offsets, offsets, (size_t)(E + 1) * 4));
    HIPCHK(tap_copy(tp.bucket_ids, ids, (size_t)T_ * 4));
  }
  HIPCHK(mark(10));
  if constexpr (std::is_same<T, bf16_t>::value) {
    HIPCHK(f8 ? launch_moe_down_f8(ma, st) : launch_moe_down<T>(ma, st));
  } else {
    HIPCHK(launch_moe_down<T>(ma, st));
  }
  HIPCHK(mark(11));
  HIPCHK(tap_copy(tp.mlp_neurons, neurons, (size_t)T_ * I * A));
  HIPCHK(tap_copy(tp.layer_output, x_out, (size_t)T_ * H * 4));
  HIPCHK(tap_copy(tp.router_state, s_out, (size_t)T_ * R * A));
  return ZAYA_OK;
}

size_t block_ws_bytes(const zaya_block_config* c, int B, int S, int decode) { return plan_block(c, B, S, decode).total; }

// Cache checks of one block call. *max_len: prefill, the largest cache_len + S; decode,
// the largest span from a sequence's 64-aligned window start to its new token.
int check_cache(const zaya_block_config* c, const zaya_cca_cache* cache, int B, int S, bool decode, int* max_len) {
  *max_len = S;
  if (!cache) return ZAYA_OK;
  if (!cache->K || !cache->V || !cache->conv_state || !cache->prev_hs || !cache->cache_len)
    return fail(ZAYA_EINVAL, "cache has a NULL member");
  if (cache->cap <= 0) return fail(ZAYA_ECACHE, "cache cap %d", cache->cap);
  const int W = c->sliding_window;
  if (cache->ring) {
    if (W < 0) return fail(ZAYA_ECACHE, "a ring cache needs a sliding window");
    if (cache->cap < W + 1) return fail(ZAYA_ECACHE, "ring cache cap %d < sliding_window + 1 = %d", cache->cap, W + 1);
  }
  int span = 1;
  for (int b = 0; b < B; ++b) {
    const int L0 = cache->cache_len[b];
    if (L0 < 0) return fail(ZAYA_ECACHE, "cache_len[%d] = %d", b, L0);
    if (cache->ring) {
      if (!decode && L0 != 0)
        return fail(ZAYA_ECACHE, "prefill into a ring cache needs fresh sequences (cache_len[%d] = %d)", b, L0);
      if (L0 > INT_MAX - S) return fail(ZAYA_ECACHE, "cache_len[%d] = %d too large", b, L0);
    } else if ((long long)L0 + S > cache->cap) {
      return fail(ZAYA_ECACHE, "cache_len[%d] = %d with S = %d exceeds cap %d", b, L0, S, cache->cap);
    }
    *max_len = std::max(*max_len, L0 + S);
    const int kbase = W >= 0 ? (std::max(0, L0 - W) / 64) * 64 : 0;
    span = std::max(span, L0 + 1 - kbase);
  }
  if (decode) *max_len = span;
  return ZAYA_OK;
}

int block_entry(const zaya_block_config* c, const zaya_block_weights* w, int B, int S, bool decode, const float* x,
                const void* s_in, float* x_out, void* s_out, const zaya_cca_cache* cache, const zaya_taps* taps,
                void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  int rc = check_config(c);
  if (rc) return rc;
  if ((rc = check_weights(c, w))) return rc;
  if (B <= 0 || S <= 0) return fail(ZAYA_EINVAL, "B=%d S=%d must be positive", B, S);
  if (decode && S != 1) return fail(ZAYA_EINVAL, "decode needs S == 1");
  if (!x || !x_out || !s_out) return fail(ZAYA_EINVAL, "x, x_out and router_state_out are required");
  if (decode && !cache) return fail(ZAYA_EINVAL, "decode needs a cache");
  const size_t T_ = (size_t)B * S;
  const size_t A = act_bytes(c);
  if (overlap(x, T_ * c->hidden * 4, x_out, T_ * c->hidden * 4)) return fail(ZAYA_EALIAS, "x_out aliases x");
  if (overlap(s_in, T_ * c->router_hidden * A, s_out, T_ * c->router_hidden * A))
    return fail(ZAYA_EALIAS, "router_state_out aliases router_state_in");
  int max_len = S;
  if ((rc = check_cache(c, cache, B, S, decode, &max_len))) return rc;
  const size_t need = block_ws_bytes(c, B, S, decode);
  if (!ws || ws_bytes < need) return fail(ZAYA_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  if (((uintptr_t)ws) & 255) return fail(ZAYA_EWORKSPACE, "workspace not 256-byte aligned");
  Plan p = plan_block(c, B, S, decode);
  hipStream_t st = (hipStream_t)stream;
  if (c->act_dtype == ZAYA_BF16)
    return run_block<bf16_t>(c, w, B, S, decode, x, s_in, x_out, s_out, cache, taps, (char*)ws, p, max_len, st);
  return run_block<float>(c, w, B, S, decode, x, s_in, x_out, s_out, cache, taps, (char*)ws, p, max_len, st);
}

// Block l's configuration in a stack: with window_layers 1 (2) only the even (odd)
// blocks keep block.sliding_window, the others attend to the whole prefix.
zaya_block_config layer_config(const zaya_stack_config* s, int l) {
  zaya_block_config c = s->block;
  if ((s->window_layers == 1 && (l & 1)) || (s->window_layers == 2 && !(l & 1))) c.sliding_window = -1;
  return c;
}

// Stack workspace: the block workspace, then two fp32 streams, two router states and
// the final normed stream.
struct StackPlan {
  size_t block, block_bytes, x0, x1, s0, s1, xf, total;
};

StackPlan plan_stack(const zaya_stack_config* c, int B, int S) {
  StackPlan p{};
  const size_t T_ = (size_t)B * S;
  const size_t A = act_bytes(&c->block);
  p.block = 0;
  // the largest block workspace over the layers' configurations (windowed or not)
  const zaya_block_config l0 = layer_config(c, 0), l1 = layer_config(c, 1);
  p.block_bytes = std::max(block_ws_bytes(&l0, B, S, 0), block_ws_bytes(&l1, B, S, 0));
  size_t o = align256(p.block_bytes);
  auto take = [&](size_t bytes) {
    size_t at = o;
    o += align256(bytes);
    return at;
  };
  p.x0 = take(T_ * c->block.hidden * 4);
  p.x1 = take(T_ * c->block.hidden * 4);
  p.s0 = take(T_ * c->block.router_hidden * A);
  p.s1 = take(T_ * c->block.router_hidden * A);
  p.xf = take(T_ * c->block.hidden * A);
  p.total = o;
  return p;
}

// ---- allocation-free decode: the workspace is a static device array. Each device the
// library runs on holds its own copy from the first use until the process ends; its
// device address comes from hipGetSymbolAddress on that device (the array's name in host
// code is only a host-side stand-in) and is kept per device.
constexpr size_t kScratchBytes = ZAYA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch array's device address on the current device, looked up on the first
// call on that device (with the device current).
int scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(ZAYA_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(ZAYA_EHIP, "device %d: only devices 0..%d are served", dev,
                                                  kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(ZAYA_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ZAYA_OK;
}

}  // namespace

extern "C" {

size_t zaya_block_workspace_bytes(const zaya_block_config* cfg, int B, int S, int decode) {
  if (check_config(cfg) || B <= 0 || S <= 0 || (decode && S != 1)) return 0;
  return block_ws_bytes(cfg, B, S, decode);
}

int zaya_block_prefill(const zaya_block_config* cfg, const zaya_block_weights* w, int B, int S, const float* x,
                       const void* router_state_in, float* x_out, void* router_state_out, const zaya_cca_cache* cache,
                       const zaya_taps* taps, void* workspace, size_t workspace_bytes, void* stream) {
  return block_entry(cfg, w, B, S, false, x, router_state_in, x_out, router_state_out, cache, taps, workspace,
                     workspace_bytes, stream);
}

int zaya_block_decode(const zaya_block_config* cfg, const zaya_block_weights* w, int B, const float* x,
                      const void* router_state_in, float* x_out, void* router_state_out, const zaya_cca_cache* cache,
                      const zaya_taps* taps, void* workspace, size_t workspace_bytes, void* stream) {
  return block_entry(cfg, w, B, 1, true, x, router_state_in, x_out, router_state_out, cache, taps, workspace,
                     workspace_bytes, stream);
}

int zaya_block_decode_noalloc(const zaya_block_config* cfg, const zaya_block_weights* w, int B, const float* x,
                              const void* router_state_in, float* x_out, void* router_state_out,
                              const zaya_cca_cache* cache, const zaya_taps* taps, void* stream) {
  g_err.clear();
  int rc = check_config(cfg);
  if (rc) return rc;
  if (B <= 0) return fail(ZAYA_EINVAL, "B=%d must be positive", B);
  const size_t need = block_ws_bytes(cfg, B, 1, 1);
  if (need > kScratchBytes)
    return fail(ZAYA_EWORKSPACE, "a decode step of %d sequences needs %zu bytes of scratch; the static array holds %zu",
                B, need, kScratchBytes);
  void* ws = nullptr;
  if ((rc = scratch_for_current_device(&ws))) return rc;
  return block_entry(cfg, w, B, 1, true, x, router_state_in, x_out, router_state_out, cache, taps, ws, kScratchBytes,
                     stream);
}

size_t zaya_stack_workspace_bytes(const zaya_stack_config* cfg, int B, int S) {
  if (!cfg || check_config(&cfg->block) || B <= 0 || S <= 0 || cfg->window_layers < 0 || cfg->window_layers > 2 ||
      cfg->n_layers <= 0 || cfg->vocab <= 0 || cfg->vocab % 4)
    return 0;
  return plan_stack(cfg, B, S).total;
}

int zaya_stack_forward(const zaya_stack_config* cfg, const zaya_stack_weights* w, int B, int S, const int32_t* ids,
                       void* logits, const zaya_cca_cache* caches, const zaya_taps* taps, void* workspace,
                       size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (!cfg) return fail(ZAYA_EINVAL, "config is NULL");
  int rc = check_config(&cfg->block);
  if (rc) return rc;
  if (cfg->n_layers <= 0 || cfg->vocab <= 0) return fail(ZAYA_ESHAPE, "n_layers %d vocab %d", cfg->n_layers, cfg->vocab);
  // the lm_head GEMM stores four logits per lane: rows must hold whole, aligned groups
  if (cfg->vocab % 4) return fail(ZAYA_ESHAPE, "vocab %d must be a multiple of 4", cfg->vocab);
  if (!w || !w->embed || !w->emb_shift || !w->emb_scale || !w->final_g || !w->blocks)
    return fail(ZAYA_EINVAL, "stack weights incomplete");
  for (int l = 0; l < cfg->n_layers; ++l)
    if ((rc = check_weights(&cfg->block, &w->blocks[l]))) return fail(rc, "block %d: %s", l, g_err.c_str());
  if (B <= 0 || S <= 0) return fail(ZAYA_EINVAL, "B=%d S=%d must be positive", B, S);
  if (!ids || !logits) return fail(ZAYA_EINVAL, "ids and logits are required");
  if (cfg->window_layers < 0 || cfg->window_layers > 2)
    return fail(ZAYA_ESHAPE, "window_layers %d not in {0, 1, 2}", cfg->window_layers);
  if (caches) {
    for (int l = 0; l < cfg->n_layers; ++l) {
      const zaya_block_config lc = layer_config(cfg, l);
      int ml;
      if ((rc = check_cache(&lc, &caches[l], B, S, false, &ml))) return fail(rc, "block %d: %s", l, g_err.c_str());
    }
  }
  StackPlan p = plan_stack(cfg, B, S);
  if (!workspace || workspace_bytes < p.total)
    return fail(ZAYA_EWORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, p.total);
  if (((uintptr_t)workspace) & 255) return fail(ZAYA_EWORKSPACE, "workspace not 256-byte aligned");
  const zaya_block_config* c = &cfg->block;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const int T_ = B * S, H = c->hidden;
  float* xs[2] = {(float*)(ws + p.x0), (float*)(ws + p.x1)};
  void* ss[2] = {ws + p.s0, ws + p.s1};
  const bool bf = c->act_dtype == ZAYA_BF16;
  hipError_t e = bf ? launch_embed<bf16_t>(ids, (const bf16_t*)w->embed, (const bf16_t*)w->emb_shift,
                                           (const bf16_t*)w->emb_scale, xs[0], nullptr, T_, H, cfg->vocab, st)
                    : launch_embed<float>(ids, (const float*)w->embed, (const float*)w->emb_shift,
                                          (const float*)w->emb_scale, xs[0], nullptr, T_, H, cfg->vocab, st);
  if (e != hipSuccess) return fail(ZAYA_EHIP, "embed: %s", hipGetErrorString(e));
  const size_t bws = p.block_bytes;
  const void* s_in = nullptr;
  int cur = 0;
  for (int l = 0; l < cfg->n_layers; ++l) {
    const zaya_cca_cache* cc = caches ? &caches[l] : nullptr;
    const zaya_taps* tt = taps ? &taps[l] : nullptr;
    const zaya_block_config lc = layer_config(cfg, l);
    rc = block_entry(&lc, &w->blocks[l], B, S, false, xs[cur], s_in, xs[cur ^ 1], ss[cur], cc, tt, ws, bws, stream);
    if (rc) return fail(rc, "block %d: %s", l, g_err.c_str());
    s_in = ss[cur];
    cur ^= 1;
  }
  void* xf = ws + p.xf;
  if (bf) {
    e = launch_rmsnorm_stream<bf16_t>(xs[cur], (const bf16_t*)w->final_g, (bf16_t*)xf, T_, H, c->rms_eps, st);
    if (e == hipSuccess)
      e = launch_gemm_store<bf16_t>((const bf16_t*)xf, H, (const bf16_t*)w->embed, H, T_, cfg->vocab, H,
                                    (bf16_t*)logits, cfg->vocab, nullptr, 0, st);
  } else {
    e = launch_rmsnorm_stream<float>(xs[cur], (const float*)w->final_g, (float*)xf, T_, H, c->rms_eps, st);
    if (e == hipSuccess)
      e = launch_gemm_store<float>((const float*)xf, H, (const float*)w->embed, H, T_, cfg->vocab, H,
                                   (float*)logits, cfg->vocab, nullptr, 0, st);
  }
  if (e != hipSuccess) return fail(ZAYA_EHIP, "final norm / lm_head: %s", hipGetErrorString(e));
  return ZAYA_OK;
}

int zaya_pack_experts(const zaya_block_config* cfg, const void* W_gu, const void* W_dn, void* W_gu_packed,
                      void* W_dn_packed, void* stream) {
  g_err.clear();
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!W_gu || !W_dn || !W_gu_packed || !W_dn_packed) return fail(ZAYA_EINVAL, "expert weight pointer is NULL");
  const int E = cfg->n_experts, H = cfg->hidden, I = cfg->expert_inter;
  const bool f8 = fp8_experts(cfg);
  const size_t A = f8 ? 1 : act_bytes(cfg);
  const size_t ngu = (size_t)E * 2 * I * H * A, ndn = (size_t)E * H * I * A;
  if (overlap(W_gu_packed, ngu, W_gu, ngu) || overlap(W_gu_packed, ngu, W_dn, ndn) ||
      overlap(W_dn_packed, ndn, W_gu, ngu) || overlap(W_dn_packed, ndn, W_dn, ndn) ||
      overlap(W_gu_packed, ngu, W_dn_packed, ndn))
    return fail(ZAYA_EALIAS, "packed expert weights overlap the row-major ones or each other");
  const hipStream_t st = (hipStream_t)stream;
  const hipError_t e =
      f8 ? launch_pack_experts_f8((const uint8_t*)W_gu, (const uint8_t*)W_dn, (uint8_t*)W_gu_packed,
                                  (uint8_t*)W_dn_packed, E, H, I, st)
      : cfg->act_dtype == ZAYA_BF16
          ? launch_pack_experts<bf16_t>((const bf16_t*)W_gu, (const bf16_t*)W_dn, (bf16_t*)W_gu_packed,
                                        (bf16_t*)W_dn_packed, E, H, I, st)
          : launch_pack_experts<float>((const float*)W_gu, (const float*)W_dn, (float*)W_gu_packed,
                                       (float*)W_dn_packed, E, H, I, st);
  if (e != hipSuccess) return fail(ZAYA_EHIP, "expert packing: %s", hipGetErrorString(e));
  return ZAYA_OK;
}

int zaya_set_stage_events(void* const* events, int n) {
  if (n == 0 || events == nullptr) {
    g_stage_events.clear();
    return ZAYA_OK;
  }
  if (n != ZAYA_N_STAGES + 1) return fail(ZAYA_EINVAL, "need %d events, got %d", ZAYA_N_STAGES + 1, n);
  g_stage_events.assign((hipEvent_t const*)events, (hipEvent_t const*)events + n);
  return ZAYA_OK;
}

const char* zaya_stage_name(int k) { return (k >= 0 && k < ZAYA_N_STAGES) ? kStageNames[k] : ""; }

const char* zaya_last_error(void) { return g_err.c_str(); }

const char* zaya_status_str(int s) {
  switch (s) {
    case ZAYA_OK: return "ZAYA_OK";
    case ZAYA_EINVAL: return "ZAYA_EINVAL";
    case ZAYA_ESHAPE: return "ZAYA_ESHAPE";
    case ZAYA_EDTYPE: return "ZAYA_EDTYPE";
    case ZAYA_EWORKSPACE: return "ZAYA_EWORKSPACE";
    case ZAYA_ECACHE: return "ZAYA_ECACHE";
    case ZAYA_EALIAS: return "ZAYA_EALIAS";
    case ZAYA_EHIP: return "ZAYA_EHIP";
    default: return "ZAYA_UNKNOWN";
  }
}

int zaya_abi_version(void) { return ZAYA_ABI_VERSION; }

}  // extern "C"
