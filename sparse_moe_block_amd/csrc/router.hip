// Router MLP, top-1 selection beside the skip class, and the merge of skip tokens.
//
// ("One expert per token, chosen beside a skip class" and the family module's mixture
// paragraph on the nnterp page; "Printout": router_mlp = RMSNorm(256), fc1, fc2 with
// bias, out_proj to E+1 classes without bias, GELU with approximate='none'.)
//   z  = rnd(g * rnd(u / sqrt(mean(u^2) + eps)))
//   a1 = rnd(gelu(rnd(z W1^T + b1))),  a2 = rnd(gelu(rnd(a1 W2^T + b2)))
//   logits = rnd(a2 Wout^T)                      (router_logits; last column = skip)
//   probs  = fp32(softmax computed in fp64 over the fp32 logits)
//   class  = first argmax of fp32(probs + balancing_biases)
//   skip (class == E): index 0, weight 0; else index = class, weight = rnd(probs[class])
// A skip token runs no expert, so its MoE merge reduces to
//   out = f32(f32(h + rb) * rs) + rnd(rnd(hsb) * hss),
// which this kernel writes directly; routed tokens are written by the expert kernels.
//
// One workgroup of 8 waves per 16 tokens. fc1, fc2 and out_proj run on MFMA with the
// weight fragments read straight from global memory into registers (L2-resident:
// 2 x 128 KiB + 8.5 KiB) and the activations in LDS. Every global read the kernel
// makes (router state first, then biases, then weights) is issued at its start, so
// the whole kernel waits for memory about once; the selection runs in registers, 16
// lanes per token.
#include "common.h"
#include "kernels.h"

namespace zaya {

constexpr int kRouterTok = 16;
constexpr int kRouterR = 256;
constexpr int kRouterWaves = 8;
constexpr int kRouterRows = kRouterR / kRouterWaves;  // fc output rows per wave

// The wave's 32 weight rows of fc1 or fc2 (its whole K range) as MFMA fragments, and
// the matching 8 bias values of this lane.
template <typename T>
struct RouterFcFrags {
  typename Mfma<T>::frag f[kRouterRows / 16][kRouterR / 32];
  float b[kRouterRows / 16][4];
  __device__ __forceinline__ void load_bias(const T* __restrict__ bias) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int nb = 0; nb < kRouterRows / 16; ++nb) load4(bias + wave * kRouterRows + nb * 16 + (lane >> 4) * 4, b[nb]);
  }
  __device__ __forceinline__ void load(const T* __restrict__ W) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int nb = 0; nb < kRouterRows / 16; ++nb)
#pragma unroll
      for (int ks = 0; ks < kRouterR / 32; ++ks)
        f[nb][ks] = Mfma<T>::load(W + (size_t)(wave * kRouterRows + nb * 16 + r16) * kRouterR + ks * 32 + grp * 8);
  }
};

template <typename T>
__device__ __forceinline__ void router_fc(const RouterFcFrags<T>& W, const T* in_s, T* out_s, int ldsrow) {
  // out[t][n] = rnd(gelu(rnd(sum_k in[t][k] W[n][k] + b[n]))), t < 16, n < 256.
  using MF = Mfma<T>;
  constexpr int KS = kRouterR / 32, NB = kRouterRows / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, grp = lane >> 4;
  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const typename MF::frag xf = MF::load(in_s + r16 * ldsrow + ks * 32 + grp * 8);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = MF::mma(W.f[nb][ks], xf, acc[nb]);
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n0 = wave * kRouterRows + nb * 16 + grp * 4;
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = Act<T>::rnd(acc[nb][i] + W.b[nb][i]);
      v[i] = Act<T>::rnd(0.5f * x * (1.0f + erff(x * 0.70710678118654752f)));
    }
    store4(out_s + r16 * ldsrow + n0, v);
  }
}

// Selection for one token: lanes 16 g .. 16 g + 15 of a wave hold the token's classes
// c = lane % 16 and 16 + lane % 16. Softmax in fp64 over the fp32 logits (max and sum by
// shuffles inside the 16-lane group), probabilities rounded to fp32, plus the balancing
// biases in fp32; the first (lowest-index) maximum wins.
__device__ __forceinline__ double group16_max(double v) {
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, 16));
  return v;
}
__device__ __forceinline__ double group16_sum(double v) {
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) v += __shfl_xor(v, o, 16);
  return v;
}

template <typename T>
__global__ __launch_bounds__(kRouterWaves * 64) void router_kernel(RouterArgs<T> a) {
  constexpr int ROW = kRouterR + 16 / (int)sizeof(T);  // padded LDS row (elements)
  __shared__ __attribute__((aligned(16))) T z_s[kRouterTok * ROW];
  __shared__ __attribute__((aligned(16))) T a1_s[kRouterTok * ROW];
  __shared__ __attribute__((aligned(16))) T a2_s[kRouterTok * ROW];
  __shared__ float lg_s[kRouterTok][33];
  __shared__ int cls_s[kRouterTok];

  const int tok0 = blockIdx.x * kRouterTok;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, grp = lane >> 4;
  const int E = a.E, NC = a.E + 1;

  // All global reads, in the order they are needed: the router state rows (wave w
  // normalizes tokens 2w, 2w+1; lane owns 4 consecutive values) and the norm gain, the
  // biases and balancing biases, then the weight fragments of fc1, fc2 and out_proj
  // (waves 0 and 1: classes 16 w .. 16 w + 15; rows past the last class repeat it and
  // are discarded).
  float v[2][4], g[4];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int tok = tok0 + wave * 2 + tt;
#pragma unroll
    for (int c = 0; c < 4; ++c) v[tt][c] = 0.f;
    if (tok < a.ntok) load4(a.u + (size_t)tok * kRouterR + lane * 4, v[tt]);
  }
  load4(a.norm_g + lane * 4, g);
  RouterFcFrags<T> w1, w2;
  w1.load_bias(a.b1);
  w2.load_bias(a.b2);
  const float bb1 = r16 < NC ? a.bal_bias[r16] : 0.f;
  const float bb2 = 16 + r16 < NC ? a.bal_bias[16 + r16] : 0.f;
  w1.load(a.W1);
  if constexpr (sizeof(T) == 2) w2.load(a.W2);  // fp32 fragments are twice the size: loaded after fc1
  typename Mfma<T>::frag wo[kRouterR / 32];
  if (wave < 2) {
    const int c = min(wave * 16 + r16, NC - 1);
#pragma unroll
    for (int ks = 0; ks < kRouterR / 32; ++ks)
      wo[ks] = Mfma<T>::load(a.Wout + (size_t)c * kRouterR + ks * 32 + grp * 8);
  }

  // RMSNorm of u
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    float ss = v[tt][0] * v[tt][0] + v[tt][1] * v[tt][1] + v[tt][2] * v[tt][2] + v[tt][3] * v[tt][3];
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)kRouterR + a.eps);
    float o[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] = Act<T>::rnd(g[c] * Act<T>::rnd(v[tt][c] * inv));
    store4(z_s + (wave * 2 + tt) * ROW + lane * 4, o);
  }
  __syncthreads();
  router_fc<T>(w1, z_s, a1_s, ROW);
  if constexpr (sizeof(T) == 4) w2.load(a.W2);
  __syncthreads();
  router_fc<T>(w2, a1_s, a2_s, ROW);
  __syncthreads();

  // out_proj on MFMA: logits[t][c] = rnd(sum_k a2[t][k] Wout[c][k]), waves 0 and 1
  if (wave < 2) {
    using MF = Mfma<T>;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kRouterR / 32; ++ks)
      acc = MF::mma(wo[ks], MF::load(a2_s + r16 * ROW + ks * 32 + grp * 8), acc);
    // lane holds classes 16 w + 4 grp + i of token r16
    const int tok = tok0 + r16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = wave * 16 + grp * 4 + i;
      const float l = Act<T>::rnd(acc[i]);
      lg_s[r16][c] = l;
      if (c < NC && tok < a.ntok) a.logits[(size_t)tok * NC + c] = Act<T>::cvt(l);
    }
  }
  __syncthreads();

  // selection: waves 0..3, wave w handles tokens 4 w .. 4 w + 3, one per 16-lane group
  if (wave < 4) {
    const int t = wave * 4 + grp, tok = tok0 + t;
    const int c1 = r16, c2 = 16 + r16;
    const bool has1 = c1 < NC, has2 = c2 < NC;  // classes past E are padding
    const double l1 = has1 ? (double)lg_s[t][c1] : -INFINITY, l2 = has2 ? (double)lg_s[t][c2] : -INFINITY;
    const double mx = group16_max(fmax(l1, l2));
    const double e1 = has1 ? exp(l1 - mx) : 0.0, e2 = has2 ? exp(l2 - mx) : 0.0;
    const double sum = group16_sum(e1 + e2);
    const float p1 = (float)(e1 / sum), p2 = (float)(e2 / sum);
    const float s1 = has1 ? p1 + bb1 : -INFINITY;
    const float s2 = has2 ? p2 + bb2 : -INFINITY;
    // best of this lane's two (c1 < c2: c2 wins only if strictly larger)
    float bs = s1, bp = p1;
    int bc = c1;
    if (s2 > s1) { bs = s2; bp = p2; bc = c2; }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) {
      const float os = __shfl_xor(bs, o, 16), op = __shfl_xor(bp, o, 16);
      const int oc = __shfl_xor(bc, o, 16);
      if (os > bs || (os == bs && oc < bc)) { bs = os; bp = op; bc = oc; }
    }
    if (r16 == 0) {
      cls_s[t] = bc;
      if (tok < a.ntok) {
        const bool skip = bc == E;
        a.cls[tok] = bc;
        a.idx[tok] = skip ? 0 : bc;
        a.wts[tok] = Act<T>::cvt(skip ? 0.f : bp);
      }
    }
  }
  __syncthreads();

  // skip tokens: out = (h + rb) * rs + rnd(rnd(hsb) * hss)
  for (int t = 0; t < kRouterTok; ++t) {
    const int tok = tok0 + t;
    if (tok >= a.ntok || cls_s[t] != E) continue;
    for (int c0 = threadIdx.x * 4; c0 < a.H; c0 += blockDim.x * 4) {
      float hv[4], b1[4], s1[4], b2[4], s2[4], mo[4], o[4];
      load4(a.h + (size_t)tok * a.H + c0, hv);
      load4(a.m_hsb + c0, b1);
      load4(a.m_hss + c0, s1);
      load4(a.m_rb + c0, b2);
      load4(a.m_rs + c0, s2);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        mo[c] = Act<T>::rnd(Act<T>::rnd(b1[c]) * s1[c]);
        o[c] = fadd(fmul(fadd(hv[c], b2[c]), s2[c]), mo[c]);
      }
      store4(a.out + (size_t)tok * a.H + c0, o);
      if (a.mlp_tap) store4(a.mlp_tap + (size_t)tok * a.H + c0, mo);
      if (a.routed_tap) {
        const float z[4] = {0.f, 0.f, 0.f, 0.f};
        store4(a.routed_tap + (size_t)tok * a.H + c0, z);
      }
    }
  }
}

template <typename T>
hipError_t launch_router(const RouterArgs<T>& a, hipStream_t s) {
  if (a.ntok <= 0) return hipSuccess;
  hipLaunchKernelGGL(router_kernel<T>, dim3((a.ntok + kRouterTok - 1) / kRouterTok), dim3(kRouterWaves * 64), 0, s,
                     a);
  return hipGetLastError();
}

template hipError_t launch_router<bf16_t>(const RouterArgs<bf16_t>&, hipStream_t);
template hipError_t launch_router<float>(const RouterArgs<float>&, hipStream_t);

}  // namespace zaya
