// Dense NT GEMMs of the block with their fused epilogues.
//
//  * store:     C = rnd(A B^T)                               (q/k/v projections; lm_head)
//  * merge:     o = rnd(A W_o^T); attention_output = rnd(rnd(o + hsb) * hss);
//               h = f32(f32(x + rb) * rs) + attention_output  (ZayaResidualScaling: "The
//               Notes / The block, in order" and "The contributions are the merges' scaled
//               terms" on the nnterp page)
//  * router_in: u = rnd(A W_d^T + b_d); with a carried state u = rnd(u + rnd(rss * s_in))
//               (router down_proj plus the previous block's state times
//               router_states_scale: "One expert per token, chosen beside a skip class")
#include "common.h"
#include "gemm_core.h"
#include "kernels.h"

namespace zaya {

template <typename T>
struct EpiStore {
  T* C;
  int ldc;
  __device__ __forceinline__ void operator()(int m, int n, const float* v) const { store4(C + (size_t)m * ldc + n, v); }
};

template <typename T>
struct EpiMerge {
  const float* x;
  const T *hsb, *hss, *rb, *rs;
  float* h;
  T* a_tap;
  int H;
  __device__ __forceinline__ void operator()(int m, int n, const float* v) const {
    float xs[4], b1[4], s1[4], b2[4], s2[4], a[4], o[4];
    load4(x + (size_t)m * H + n, xs);
    load4(hsb + n, b1);
    load4(hss + n, s1);
    load4(rb + n, b2);
    load4(rs + n, s2);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float oc = Act<T>::rnd(v[c]);
      a[c] = Act<T>::rnd(Act<T>::rnd(oc + b1[c]) * s1[c]);
      o[c] = fadd(fmul(fadd(xs[c], b2[c]), s2[c]), a[c]);
    }
    store4(h + (size_t)m * H + n, o);
    if (a_tap) store4(a_tap + (size_t)m * H + n, a);
  }
};

template <typename T>
struct EpiRouterIn {
  const T* b;
  const T* rss;
  const T* s_in;  // NULL: block-0 semantics
  T* u;
  int R;
  __device__ __forceinline__ void operator()(int m, int n, const float* v) const {
    float bb[4], o[4];
    load4(b + n, bb);
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] = Act<T>::rnd(v[c] + bb[c]);
    if (s_in) {
      float sc[4], st[4];
      load4(rss + n, sc);
      load4(s_in + (size_t)m * R + n, st);
#pragma unroll
      for (int c = 0; c < 4; ++c) o[c] = Act<T>::rnd(o[c] + Act<T>::rnd(sc[c] * st[c]));
    }
    store4(u + (size_t)m * R + n, o);
  }
};

template <typename T, int BM, int BN, int WM, int WN, class Epi>
__global__ __launch_bounds__(WM* WN * 64) void gemm_nt_kernel(const T* __restrict__ A, int lda, const T* __restrict__ B,
                                                               int ldb, int M, int N, int K, Epi epi) {
  using Tile = GemmTile<T, BM, BN, WM, WN>;
  __shared__ __attribute__((aligned(16))) char smem[Tile::kLdsBytes];
  const int ntn = (N + BN - 1) / BN;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int m0 = (wg / ntn) * BM, n0 = (wg % ntn) * BN;
  Tile t;
  t.set_a([&](int r) -> const T* { return m0 + r < M ? A + (size_t)(m0 + r) * lda : nullptr; });
  t.set_b([&](int r) -> const T* { return n0 + r < N ? B + (size_t)(n0 + r) * ldb : nullptr; });
  t.run(smem, K / Tile::kBK);
  t.epilogue([&](int m, int n, const float* v) {
    if (m0 + m < M && n0 + n < N) epi(m0 + m, n0 + n, v);
  });
}

template <typename T, int BM, int BN, int WM, int WN, class Epi>
static hipError_t launch_cfg(const T* A, int lda, const T* B, int ldb, int M, int N, int K, Epi epi, hipStream_t s) {
  const int g = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_nt_kernel<T, BM, BN, WM, WN, Epi>), dim3(g), dim3(WM * WN * 64), 0, s, A, lda, B, ldb, M,
                     N, K, epi);
  return hipGetLastError();
}

// Tile choice: 128x128 (4 waves of 64x64) when there are enough rows, else 32x64
// (4 waves of 32x16) so weight-streaming GEMMs with few rows still spread over many CUs.
template <typename T, class Epi>
static hipError_t launch_any(const T* A, int lda, const T* B, int ldb, int M, int N, int K, Epi epi, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (M >= 512) return launch_cfg<T, 128, 128, 2, 2>(A, lda, B, ldb, M, N, K, epi, s);
  return launch_cfg<T, 32, 64, 1, 4>(A, lda, B, ldb, M, N, K, epi, s);
}

template <typename T>
hipError_t launch_gemm_store(const T* A, int lda, const T* B, int ldb, int M, int N, int K, T* C, int ldc,
                             hipStream_t s) {
  return launch_any(A, lda, B, ldb, M, N, K, EpiStore<T>{C, ldc}, s);
}

template <typename T>
hipError_t launch_gemm_merge(const T* O, const T* Wo, int M, int H, int K, const float* x, const T* hsb, const T* hss,
                             const T* rb, const T* rs, float* h, T* a_tap, hipStream_t s) {
  return launch_any(O, K, Wo, K, M, H, K, EpiMerge<T>{x, hsb, hss, rb, rs, h, a_tap, H}, s);
}

template <typename T>
hipError_t launch_gemm_router_in(const T* hn, const T* Wd, int M, int R, int H, const T* b, const T* rss,
                                 const T* s_in, T* u, hipStream_t s) {
  return launch_any(hn, H, Wd, H, M, R, H, EpiRouterIn<T>{b, rss, s_in, u, R}, s);
}

#define ZAYA_INST(T)                                                                                                 \
  template hipError_t launch_gemm_store<T>(const T*, int, const T*, int, int, int, int, T*, int, hipStream_t);       \
  template hipError_t launch_gemm_merge<T>(const T*, const T*, int, int, int, const float*, const T*, const T*,      \
                                           const T*, const T*, float*, T*, hipStream_t);                             \
  template hipError_t launch_gemm_router_in<T>(const T*, const T*, int, int, int, const T*, const T*, const T*, T*, \
                                               hipStream_t);
ZAYA_INST(bf16_t)
ZAYA_INST(float)
#undef ZAYA_INST

}  // namespace zaya
