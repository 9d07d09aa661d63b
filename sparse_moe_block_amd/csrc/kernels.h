// Internal launch interface between the C ABI (zaya_api.cpp) and the kernels.
// Every launcher enqueues on the given stream and returns hipGetLastError().
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"

namespace zaya {

// ---- norms / embedding
template <typename T>
hipError_t launch_rmsnorm_stream(const float* x, const T* g, T* out, int rows, int H, float eps, hipStream_t s);
template <typename T>
hipError_t launch_embed(const int32_t* ids, const T* table, const T* shift, const T* scale, float* x0, T* tap,
                        int rows, int H, int vocab, hipStream_t s);

// ---- dense GEMMs (A [M,K] rows, B [N,K] rows). part/part_bytes: fp32 scratch for the
// split-K path taken when M <= 64 (NULL: no split).
template <typename T>
hipError_t launch_gemm_store(const T* A, int lda, const T* B, int ldb, int M, int N, int K, T* C, int ldc,
                             float* part, size_t part_bytes, hipStream_t s);
// Decode helpers (at most 64 rows). Two store GEMMs with the same K in one split-K pass
// and one reduction pass (two plain launches when a split does not pay).
template <typename T>
hipError_t launch_gemm_store_pair(const T* A1, int lda1, const T* B1, int ldb1, int M1, int N1, T* C1, int ldc1,
                                  const T* A2, int lda2, const T* B2, int ldb2, int M2, int N2, T* C2, int ldc2, int K,
                                  float* part, size_t part_bytes, hipStream_t s);
// Only the split-K partial products [kparts][M][N] into part; returns kparts (> 1), 0 when
// the GEMM is not split (nothing launched), -1 on a launch error.
template <typename T>
int launch_gemm_parts(const T* A, int lda, const T* B, int ldb, int M, int N, int K, float* part, size_t part_bytes,
                      hipStream_t s);
// Only the split-K partial products of a pair of GEMMs with the same K (as
// launch_gemm_store_pair): [kparts][M1][N1] at part, then [kparts][M2][N2]; returns
// kparts (> 1), 0 when not split (nothing launched), -1 on a launch error. The consumer
// sums the parts in ascending order from zero and rounds, as the pair's reduction would.
template <typename T>
int launch_gemm_pair_parts(const T* A1, int lda1, const T* B1, int ldb1, int M1, int N1, const T* A2, int lda2,
                           const T* B2, int ldb2, int M2, int N2, int K, float* part, size_t part_bytes, hipStream_t s);
// Sum of the o_proj partials, the attention merge (as the merge epilogue) and the
// post-attention RMSNorm of the result, one wave per row: writes h (and the
// attention_output tap) and hn.
template <typename T>
hipError_t launch_merge_norm_parts(const float* part, int kparts, int rows, int H, const float* x, const T* hsb,
                                   const T* hss, const T* rb, const T* rs, float* h, T* a_tap, const T* g2, T* hn,
                                   float eps, hipStream_t s);
template <typename T>
hipError_t launch_gemm_merge(const T* O, const T* Wo, int M, int H, int K, const float* x, const T* hsb, const T* hss,
                             const T* rb, const T* rs, float* h, T* a_tap, float* part, size_t part_bytes,
                             hipStream_t s);
template <typename T>
hipError_t launch_gemm_router_in(const T* hn, const T* Wd, int M, int R, int H, const T* b, const T* rss,
                                 const T* s_in, T* u, float* part, size_t part_bytes, hipStream_t s);

// ---- CCA projection
template <typename T>
struct CcaArgs {
  const T* P;  // [T, qkv_ld] projections of every new token
  int qkv_ld;
  const T* vdp;  // [B, nkv*d/2] prev_hs @ W_vd^T
  const T* conv_w;
  const T* conv_b;
  const T* temp;
  T* conv_state;  // [B, C, 2] in/out
  T* prev_hs;     // [B, H] out
  const T* xn;    // [T, H] normed input (source of the new prev_hs)
  const int32_t* cache_len;  // device [B]
  T* Q;  // [T, nh, d]
  T* K;  // [B, nkv, cap, d]
  T* V;
  int cap;
  T* q_tap;  // [B, nh, S, d] or NULL
  T* k_tap;  // [B, nkv, S, d] or NULL
  T* v_tap;
  int B, S, H, nh, nkv, d, rope_dim, C;
  float theta;
  int conv_k = 3;         // 3: one depthwise conv; 2: depthwise k2 then grouped k2
  const T* y2 = nullptr;  // conv_k == 2: the convolved q/k channels [B*S][C] (launch_conv2)
  int ring = 0;           // K/V slot of position p: p % cap (else p)
  // Decode with the kernel-3 conv: P and vdp are not formed; the kernel sums the q/k/v
  // projection's split-K partials ([kparts][B*S][qkv_ld]) and the delayed value's
  // ([kparts][B][nkv*d/2]) itself and rounds them (one tile per sequence: S <= 16).
  const float* qkv_part = nullptr;
  const float* vd_part = nullptr;
  int kparts = 0;
};
template <typename T>
hipError_t launch_cca(const CcaArgs<T>& a, hipStream_t s);
// Store the keys and values of positions max(0, S - cap) .. S-1 of fresh sequences,
// formed in Kw/Vw [B, nkv, S, d], into ring caches K/V [B, nkv, cap, d] at slot p % cap.
template <typename T>
hipError_t launch_ring_store(const T* Kw, const T* Vw, T* K, T* V, int B, int nkv, int S, int d, int cap,
                             hipStream_t s);

// The printout's two-stage q/k convolution (conv_k == 2) of every token: depthwise
// kernel 2 (conv_w [C][2], conv_b), then grouped kernel 2 with one group per head
// (conv2_w [C][2][d], conv2_b), each output rounded to T. History from conv_state
// (slot 0 = input, slot 1 = depthwise output, one token back), zeros when fresh.
template <typename T>
struct Conv2Args {
  const T* P;  // [B*S][qkv_ld]: columns 0 .. C are the q then k channels
  int qkv_ld;
  const T* conv_w;
  const T* conv_b;
  const T* conv2_w;
  const T* conv2_b;
  const T* conv_state;  // [B][C][2]
  const int32_t* cache_len;
  T* y2;  // [B*S][C]
  int B, S, C, d;
};
template <typename T>
hipError_t launch_conv2(const Conv2Args<T>& a, hipStream_t s);
// dynamic LDS of one CCA workgroup (two: the two-stage convolution)
size_t cca_lds_bytes(int d, int G, int act_bytes, bool two);

// ---- attention
template <typename T>
struct AttnArgs {
  const T* Q;  // [B, S, nh, d]
  const T* K;  // [B, nkv, cap, d]
  const T* V;
  T* O;  // [B, S, nh, d]
  const int32_t* cache_len;  // device [B], or null: every sequence fresh
  int B, S, nh, nkv, d, cap, window;
  int ring = 0;  // decode only: position p lives in slot p % cap
};
template <typename T>
hipError_t launch_attn_prefill(const AttnArgs<T>& a, float* part, int NC, hipStream_t s);
// key tiles per prefill unit of the kernel the shape selects, and the chunk count per
// query tile that keeps units within it
int attn_prefill_chunk_tiles(int act_bytes, int d, int G);
int attn_prefill_chunks(int S, int max_cache_len, int window, int chunk_tiles);
size_t attn_prefill_part_bytes(int B, int S, int nkv, int G, int d, int NC);
template <typename T>
// span: the largest number of positions from a sequence's 64-aligned window start (0
// without a window) to its new token, over the batch
hipError_t launch_attn_decode(const AttnArgs<T>& a, float* part, int span, hipStream_t s);
size_t attn_decode_part_bytes(int B, int nkv, int G, int d);

// ---- router MLP + selection (+ skip-token merge)
template <typename T>
struct RouterArgs {
  const T* u;  // [T, R] router state after the carried-state add
  const T* norm_g;
  const T* W1;
  const T* b1;
  const T* W2;
  const T* b2;
  const T* Wout;  // [E+1, R]
  const float* bal_bias;
  T* logits;  // [T, E+1]
  int32_t* cls;
  int32_t* idx;
  T* wts;
  const float* h;  // [T, H] stream after the attention merge
  const T* m_hsb;
  const T* m_hss;
  const T* m_rb;
  const T* m_rs;
  float* out;      // [T, H] layer output (skip tokens written here)
  T* routed_tap;   // [T, H] or NULL
  T* mlp_tap;      // [T, H] or NULL
  int ntok, R, E, H;
  float eps;
  // Few tokens: u is not formed by a reduction pass; the kernel sums the router
  // down-projection's split-K partials ([kparts][ntok][R]) itself, applies its
  // epilogue (bias, then the carried state times rss when s_in is given) and writes u_out.
  const float* part = nullptr;
  int kparts = 0;
  const T* bd = nullptr;
  const T* rss = nullptr;
  const T* s_in = nullptr;
  T* u_out = nullptr;
  // tokens of each class c in workgroup r's tile at counts[c * counts_ld + r] (for the
  // buckets), or NULL
  int32_t* counts = nullptr;
  int counts_ld = 0;
};
constexpr int kRouterTokens = 16;  // tokens per router workgroup
template <typename T>
hipError_t launch_router(const RouterArgs<T>& a, hipStream_t s);

// ---- mixture of experts
// counts: the router's per-tile class counts, class c of tile r at c * bucket_counts_ld(ntok) + r
int bucket_counts_ld(int ntok);
hipError_t launch_bucket(const int32_t* cls, const int32_t* counts, int ntok, int E, int32_t* offsets, int32_t* ids,
                         hipStream_t s);

template <typename T>
struct MoeArgs {
  const int32_t* offsets;  // [E+1]
  const int32_t* ids;      // [ntok] (first offsets[E] used)
  const T* hn;             // [ntok, H]
  const T* W_gu;           // [E, 2I, H]
  const T* W_dn;           // [E, H, I]
  T* neurons;              // [ntok, I] bucket order
  const T* wts;            // [ntok]
  const float* h;          // [ntok, H]
  const T* hsb;
  const T* hss;
  const T* rb;
  const T* rs;
  float* out;     // [ntok, H]
  T* routed_tap;  // or NULL
  T* mlp_tap;     // or NULL
  int ntok, H, I, E;
  const float* gu_scale = nullptr;  // FP8 experts: row scales [E, 2I] and [E, H]
  const float* dn_scale = nullptr;
  // At most 64 tokens: the gate/up kernel forms the buckets itself from the classes
  // (each workgroup in LDS) and workgroup 0 stores them to offsets_out / ids_out for
  // the down kernel and the taps; offsets and ids are then read only by the down kernel.
  const int32_t* cls = nullptr;
  int32_t* offsets_out = nullptr;
  int32_t* ids_out = nullptr;
  // W_gu / W_dn in the packed layout of launch_pack_experts (act-dtype experts only)
  int packed = 0;
  // workgroups resident on the device at once (set by the launchers; see moe_item)
  int slots = 0;
};
// Packed expert weights: rows in groups of kPackRows, each group stored slice after
// slice (kPackSliceBytes of every row of the group, row after row), groups of an
// expert after one another. W_gu groups hold the gate/up items' row order (see moe.hip).
constexpr int kPackRows = 128;
constexpr int kPackSliceBytes = 128;
template <typename T>
hipError_t launch_pack_experts(const T* Wgu, const T* Wdn, T* Pgu, T* Pdn, int E, int H, int I, hipStream_t s);
// FP8 codes: rows in blocks of 16, each block stored 64-byte K step after step
constexpr int kF8PackRows = 16;
constexpr int kF8PackStep = 64;
hipError_t launch_pack_experts_f8(const uint8_t* Wgu, const uint8_t* Wdn, uint8_t* Pgu, uint8_t* Pdn, int E, int H,
                                  int I, hipStream_t s);
template <typename T>
hipError_t launch_moe_gateup(const MoeArgs<T>& a, hipStream_t s);
// FP8 (E4M3) expert weights with fp32 row scales, bf16 activations
hipError_t launch_moe_gateup_f8(const MoeArgs<bf16_t>& a, hipStream_t s);
hipError_t launch_moe_down_f8(const MoeArgs<bf16_t>& a, hipStream_t s);
template <typename T>
hipError_t launch_moe_down(const MoeArgs<T>& a, hipStream_t s);

// ---- small helpers
hipError_t launch_fill_i32(int32_t* p, int n, int v, hipStream_t s);

}  // namespace zaya
