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
// One workgroup of 4 waves per 16 tokens. fc1/fc2 run on MFMA with the weights read
// straight from global memory (L2-resident: 2 x 128 KiB) and the activations in LDS.
#include "common.h"
#include "kernels.h"

namespace zaya {

constexpr int kRouterTok = 16;
constexpr int kRouterR = 256;

// The wave's 64 weight rows of fc1 or fc2 (its whole K range) as MFMA fragments.
template <typename T>
struct RouterFcFrags {
  typename Mfma<T>::frag f[4][kRouterR / 32];
  __device__ __forceinline__ void load(const T* __restrict__ W) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int ks = 0; ks < kRouterR / 32; ++ks)
        f[nb][ks] = Mfma<T>::load(W + (size_t)(wave * 64 + nb * 16 + r16) * kRouterR + ks * 32 + grp * 8);
  }
};

template <typename T>
__device__ __forceinline__ void router_fc(const RouterFcFrags<T>& W, const T* __restrict__ bias, const T* in_s,
                                          T* out_s, int ldsrow) {
  // out[t][n] = rnd(gelu(rnd(sum_k in[t][k] W[n][k] + b[n]))), t < 16, n < 256.
  using MF = Mfma<T>;
  constexpr int KS = kRouterR / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, grp = lane >> 4;
  const auto& wf = W.f;
  f32x4 acc[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const typename MF::frag xf = MF::load(in_s + r16 * ldsrow + ks * 32 + grp * 8);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[nb] = MF::mma(wf[nb][ks], xf, acc[nb]);
  }
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int n0 = wave * 64 + nb * 16 + grp * 4;
    float bb[4], v[4];
    load4(bias + n0, bb);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = Act<T>::rnd(acc[nb][i] + bb[i]);
      v[i] = Act<T>::rnd(0.5f * x * (1.0f + erff(x * 0.70710678118654752f)));
    }
    store4(out_s + r16 * ldsrow + n0, v);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void router_kernel(RouterArgs<T> a) {
  constexpr int ROW = kRouterR + 16 / (int)sizeof(T);  // padded LDS row (elements)
  __shared__ __attribute__((aligned(16))) T z_s[kRouterTok * ROW];
  __shared__ __attribute__((aligned(16))) T a1_s[kRouterTok * ROW];
  __shared__ __attribute__((aligned(16))) T a2_s[kRouterTok * ROW];
  __shared__ float lg_s[kRouterTok][64];
  __shared__ int cls_s[kRouterTok];
  __shared__ double ex_s[kRouterTok][64];
  __shared__ double mx_s[kRouterTok];
  __shared__ float bb_s[64];
  __shared__ __attribute__((aligned(16))) T wout_s[64 * ROW];  // out_proj rows, staged once

  const int tok0 = blockIdx.x * kRouterTok;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int E = a.E, NC = a.E + 1;

  // Every global tensor this kernel reads is first touched here, together, so the
  // memory round trips (and address-translation walks) of its phases overlap instead
  // of queueing one phase after another: fc1's weight fragments go straight into
  // registers, fc2's and the skip-merge parameters are touched with one load each.
  RouterFcFrags<T> w1;
  w1.load(a.W1);
  {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const T* touch[] = {a.W2 + (size_t)(wave * 64 + lane) * kRouterR, a.b1, a.b2, a.norm_g, a.m_hsb, a.m_hss,
                        a.m_rb, a.m_rs};
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc += *reinterpret_cast<const volatile uint16_t*>(touch[i]);
    if (acc == 0xFFFFFFFFu) a.cls[0] = -1;  // never true: keeps the touches alive
  }
  // stage out_proj (E+1 rows of R) and the balancing biases in LDS
  if (threadIdx.x < NC) bb_s[threadIdx.x] = a.bal_bias[threadIdx.x];
  {
    constexpr int E16 = 16 / (int)sizeof(T);
    const int nchunk = NC * (kRouterR / E16);
    for (int ch = threadIdx.x; ch < nchunk; ch += blockDim.x) {
      const int r = ch / (kRouterR / E16), col = (ch % (kRouterR / E16)) * E16;
      *reinterpret_cast<uint4*>(wout_s + r * ROW + col) =
          *reinterpret_cast<const uint4*>(a.Wout + (size_t)r * kRouterR + col);
    }
  }
  // RMSNorm of u: wave w handles tokens 4w..4w+3, lane owns 4 consecutive values; the
  // four rows are loaded together
  {
    float v[4][4], g[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int tok = tok0 + wave * 4 + tt;
#pragma unroll
      for (int c = 0; c < 4; ++c) v[tt][c] = 0.f;
      if (tok < a.ntok) load4(a.u + (size_t)tok * kRouterR + lane * 4, v[tt]);
    }
    load4(a.norm_g + lane * 4, g);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      float ss = v[tt][0] * v[tt][0] + v[tt][1] * v[tt][1] + v[tt][2] * v[tt][2] + v[tt][3] * v[tt][3];
      ss = wave_sum(ss);
      const float inv = 1.0f / sqrtf(ss / (float)kRouterR + a.eps);
      float o[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) o[c] = Act<T>::rnd(g[c] * Act<T>::rnd(v[tt][c] * inv));
      store4(z_s + (wave * 4 + tt) * ROW + lane * 4, o);
    }
  }
  __syncthreads();
  router_fc<T>(w1, a.b1, z_s, a1_s, ROW);
  RouterFcFrags<T> w2;
  w2.load(a.W2);
  __syncthreads();
  router_fc<T>(w2, a.b2, a1_s, a2_s, ROW);
  __syncthreads();

  // out_proj: (token, class) pairs
  for (int task = threadIdx.x; task < kRouterTok * NC; task += blockDim.x) {
    const int t = task / NC, c = task % NC;
    const T* wr = wout_s + c * ROW;
    const T* xr = a2_s + t * ROW;
    float acc = 0.f;
    for (int k = 0; k < kRouterR; k += 4) {
      float wv[4], xv[4];
      load4(wr + k, wv);
      load4(xr + k, xv);
      acc += wv[0] * xv[0] + wv[1] * xv[1] + wv[2] * xv[2] + wv[3] * xv[3];
    }
    const float l = Act<T>::rnd(acc);
    lg_s[t][c] = l;
    const int tok = tok0 + t;
    if (tok < a.ntok) a.logits[(size_t)tok * NC + c] = Act<T>::cvt(l);
  }
  __syncthreads();

  // selection: softmax over the fp32 logits in double, rounded to fp32 (the exponentials
  // and quotients of all (token, class) pairs in parallel), plus the balancing biases
  // in fp32, first argmax
  if (threadIdx.x < kRouterTok) {
    const int t = threadIdx.x;
    double mx = -INFINITY;
    for (int c = 0; c < NC; ++c) mx = fmax(mx, (double)lg_s[t][c]);
    mx_s[t] = mx;
  }
  __syncthreads();
  for (int task = threadIdx.x; task < kRouterTok * NC; task += blockDim.x) {
    const int t = task / NC, c = task % NC;
    ex_s[t][c] = exp((double)lg_s[t][c] - mx_s[t]);
  }
  __syncthreads();
  if (threadIdx.x < kRouterTok) {
    const int t = threadIdx.x;
    double sum = 0.0;
    for (int c = 0; c < NC; ++c) sum += ex_s[t][c];
    mx_s[t] = sum;
  }
  __syncthreads();
  for (int task = threadIdx.x; task < kRouterTok * NC; task += blockDim.x) {
    const int t = task / NC, c = task % NC;
    lg_s[t][c] = (float)(ex_s[t][c] / mx_s[t]);  // probabilities replace the logits
  }
  __syncthreads();
  if (threadIdx.x < kRouterTok) {
    const int t = threadIdx.x, tok = tok0 + t;
    int best = 0;
    float best_s = -INFINITY, best_p = 0.f;
    for (int c = 0; c < NC; ++c) {
      const float p = lg_s[t][c];
      const float sg = p + bb_s[c];
      if (sg > best_s) {
        best_s = sg;
        best = c;
        best_p = p;
      }
    }
    cls_s[t] = best;
    if (tok < a.ntok) {
      const bool skip = best == E;
      a.cls[tok] = best;
      a.idx[tok] = skip ? 0 : best;
      a.wts[tok] = Act<T>::cvt(skip ? 0.f : best_p);
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
  hipLaunchKernelGGL(router_kernel<T>, dim3((a.ntok + kRouterTok - 1) / kRouterTok), dim3(256), 0, s, a);
  return hipGetLastError();
}

template hipError_t launch_router<bf16_t>(const RouterArgs<bf16_t>&, hipStream_t);
template hipError_t launch_router<float>(const RouterArgs<float>&, hipStream_t);

}  // namespace zaya
