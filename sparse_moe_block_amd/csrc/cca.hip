// Compressed convolutional attention projection, fused (HBM-bound).
//
// From the projections P = [q | k | v_current | v_delayed] of every token
// ("Printout": ZayaCCAProjection) this kernel computes, per token t at position
// p = cache_len + t ("Queries and keys are convolved, normed to √head_dim and the keys
// scaled" on the nnterp page):
//   y_c(t)  = cb[c] + cw[c,0] x_c(t-2) + cw[c,1] x_c(t-1) + cw[c,2] x_c(t)
//             over the q and k channels (x(t<0) from conv_state, zero when fresh);
//   rq_h    = (q_h + k_g)/2,  rk_g = mean of rq_h over the query heads of group g;
//   q~ = yq + rq, k~ = yk + rk; each head scaled to length sqrt(d), keys times temp[g];
//   rotary on the first rope_dim dims (pairs (j, j + rope_dim/2), angle p*theta^(-2j/r));
//   V_g(t) = [v_current_g(t) | v_delayed_g(t-1)] (t = 0 reads prev_hs @ W_vd^T).
// Q goes to [T, nh, d]; K and V to the cache at position p; conv_state and prev_hs
// are advanced for the next call.
//
// Work split: one workgroup per (16-token tile, KV group, sequence). The tile's
// projection rows (plus two tokens of history), the group's conv taps and biases are
// first staged in LDS with coalesced 16-byte loads; then each wave takes one token at a
// time (two when d = 64). Lane p owns the dim pair (da, db) of every head of the group:
// for p < rope_dim/2 that pair is the rotary pair, so the rotation never leaves the
// lane; the head norms are reductions over the d/2 lanes of a token.
#include "common.h"
#include "kernels.h"

namespace zaya {

constexpr int kCcaTokens = 16;
constexpr int kCcaRows = kCcaTokens + 2;  // the tile plus two tokens of history

// LDS layout of one tile (act elements, row r = token t0 - 2 + r):
//   xs[r][0 .. G*d)        q channels of the group's heads
//   xs[r][G*d .. (G+1)*d)  k channels of the group's key head
//   xs[r][(G+1)*d .. +d/2) v_current half of the group
//   xs[r][.. +d/2)          v_delayed half of the group
// D (head_dim) and GG (query heads per KV head) are compile-time, so the per-head
// loops unroll and the head norms' cross-lane reductions run side by side.
template <typename T, int D, int GG>
__global__ __launch_bounds__(256) void cca_kernel(CcaArgs<T> a) {
  extern __shared__ __attribute__((aligned(16))) char cca_lds[];
  const int b = blockIdx.z, g = blockIdx.y, tile = blockIdx.x;
  constexpr int d = D, G = GG;
  const int nh = a.nh, nkv = a.nkv, r = a.rope_dim;
  const int GC = (G + 1) * d;          // q and k channels of the group
  const int ROWE = GC + d;             // + both value halves
  T* xs = reinterpret_cast<T*>(cca_lds);
  float* wsm = reinterpret_cast<float*>(cca_lds + ((kCcaRows * ROWE * (int)sizeof(T) + 15) & ~15));
  // wsm[c*4 + 0..2] = conv taps of group channel c, wsm[c*4 + 3] = its bias
  T* outs = reinterpret_cast<T*>(reinterpret_cast<char*>(wsm) + GC * 4 * sizeof(float));
  // outs: per wave, the rows of the token(s) of one step (G query heads, key, value)
  // gathered so they leave in 16-byte stores
  const int S = a.S, QR = a.qkv_ld;
  const int kcol = nh * d, vccol = nh * d + nkv * d, vdcol = vccol + nkv * d / 2;
  const int L0 = a.cache_len[b];
  const bool fresh = L0 == 0;
  const int t0 = tile * kCcaTokens;
  const int t_end = min(S, t0 + kCcaTokens);

  // group channel c -> global channel (column of P, row of conv_w / conv_state)
  auto gchan = [&](int c) { return c < G * d ? g * G * d + c : kcol + g * d + (c - G * d); };

  // the last token's normed input becomes prev_hs: requested now, stored at the end
  constexpr int E16 = 16 / (int)sizeof(T);
  const bool write_prev = t_end == S && g == 0;
  const int prev_chunks = a.H / E16;
  u32x4 prev[4];
  if (write_prev) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = threadIdx.x + k * (int)blockDim.x;
      if (i < prev_chunks) prev[k] = *reinterpret_cast<const u32x4*>(a.xn + ((size_t)b * S + S - 1) * a.H + i * E16);
    }
  }

  // 1. stage projection rows of tokens t0-2 .. t_end-1 (16-byte chunks of the four
  //    contiguous segments), the history rows from conv_state / zeros, and the conv
  //    taps. Each loop issues its loads in batches of kBatch per thread before any of
  //    them is stored, so the tile waits for memory a few times, not once per chunk.
  {
    constexpr int kBatch = 8;
    const int nthr = (int)blockDim.x;
    const int segq = G * d / E16, segk = d / E16, segv = (d / 2) / E16;
    const int per_row = segq + segk + 2 * segv;
    const int nrows = t_end - t0 + 2;
    auto chunk_cols = [&](int cc, int& src, int& dst) {
      if (cc < segq) {
        src = g * G * d + cc * E16;
        dst = cc * E16;
      } else if (cc < segq + segk) {
        src = kcol + g * d + (cc - segq) * E16;
        dst = G * d + (cc - segq) * E16;
      } else if (cc < segq + segk + segv) {
        src = vccol + g * (d / 2) + (cc - segq - segk) * E16;
        dst = GC + (cc - segq - segk) * E16;
      } else {
        src = vdcol + g * (d / 2) + (cc - segq - segk - segv) * E16;
        dst = GC + d / 2 + (cc - segq - segk - segv) * E16;
      }
    };
    for (int c0 = threadIdx.x; c0 < nrows * per_row; c0 += kBatch * nthr) {
      u32x4 val[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const int ch = c0 + k * nthr;
        const int rr = ch / per_row, t = t0 - 2 + rr;
        int src, dst;
        chunk_cols(ch % per_row, src, dst);
        if (ch < nrows * per_row && t >= 0)  // rows before the sequence start are the history
          val[k] = *reinterpret_cast<const u32x4*>(a.P + ((size_t)b * S + t) * QR + src);
      }
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const int ch = c0 + k * nthr;
        const int rr = ch / per_row, t = t0 - 2 + rr;
        int src, dst;
        chunk_cols(ch % per_row, src, dst);
        if (ch < nrows * per_row && t >= 0) *reinterpret_cast<u32x4*>(xs + rr * ROWE + dst) = val[k];
      }
    }
    // history (tokens -2, -1 of a sequence with cached tokens): q/k channels from
    // conv_state, the delayed value from prev_hs @ W_vd^T
    if (t0 == 0) {
      for (int i0 = threadIdx.x; i0 < 2 * GC; i0 += kBatch * nthr) {
        T hv[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          const int i = i0 + k * nthr;
          const int rr = i / GC, c = i % GC;
          hv[k] = (fresh || i >= 2 * GC) ? Act<T>::cvt(0.f) : a.conv_state[((size_t)b * a.C + gchan(c)) * 2 + rr];
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          const int i = i0 + k * nthr;
          if (i < 2 * GC) xs[(i / GC) * ROWE + i % GC] = hv[k];
        }
      }
      for (int i = threadIdx.x; i < d / 2; i += nthr)
        xs[1 * ROWE + GC + d / 2 + i] =
            fresh ? Act<T>::cvt(0.f) : a.vdp[(size_t)b * (nkv * d / 2) + g * (d / 2) + i];
    }
    for (int c0 = threadIdx.x; c0 < GC; c0 += 2 * nthr) {
      float wv[2][4];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int c = c0 + k * nthr;
        const int gc = gchan(min(c, GC - 1));
        wv[k][0] = Act<T>::tof(a.conv_w[gc * 3 + 0]);
        wv[k][1] = Act<T>::tof(a.conv_w[gc * 3 + 1]);
        wv[k][2] = Act<T>::tof(a.conv_w[gc * 3 + 2]);
        wv[k][3] = Act<T>::tof(a.conv_b[gc]);
      }
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int c = c0 + k * nthr;
        if (c < GC)
#pragma unroll
          for (int q = 0; q < 4; ++q) wsm[c * 4 + q] = wv[k][q];
      }
    }
  }
  __syncthreads();

  // 2. compute: lane p owns the dim pair (da, db) of every head of the group
  constexpr int spt = d / 2;     // lanes per token
  constexpr int tpw = 64 / spt;  // tokens per wave step
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane / spt, p = lane % spt;
  const int da = p < r / 2 ? p : r + (p - r / 2);
  const int db = p < r / 2 ? p + r / 2 : r + (d - r) / 2 + (p - r / 2);
  const float sqrt_d = sqrtf((float)d);
  const float temp = Act<T>::tof(a.temp[g]);
  const double inv_freq = p < r / 2 ? pow((double)a.theta, -2.0 * (double)p / (double)r) : 0.0;
  for (int base = t0 + wave * tpw; base < t_end; base += 4 * tpw) {
    const int t = base + sub;
    const bool active = t < t_end;
    const int tt = active ? t : t_end - 1;
    const int rr = tt - t0 + 2;  // LDS row of token tt
    const T* x0 = xs + rr * ROWE;  // t
    const T* x1 = x0 - ROWE;       // t - 1
    const T* x2 = x1 - ROWE;       // t - 2
    auto conv = [&](int c) -> float {
      const float* w = wsm + c * 4;
      return w[3] + w[0] * Act<T>::tof(x2[c]) + w[1] * Act<T>::tof(x1[c]) + w[2] * Act<T>::tof(x0[c]);
    };
    const int kca = G * d + da, kcb = G * d + db;
    const float pka = Act<T>::tof(x0[kca]), pkb = Act<T>::tof(x0[kcb]);
    float qa[G], qb[G];
    float rka = 0.f, rkb = 0.f;
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const int ca = hh * d + da, cb = hh * d + db;
      const float rqa = (Act<T>::tof(x0[ca]) + pka) * 0.5f, rqb = (Act<T>::tof(x0[cb]) + pkb) * 0.5f;
      rka += rqa;
      rkb += rqb;
      qa[hh] = conv(ca) + rqa;
      qb[hh] = conv(cb) + rqb;
    }
    const float ka = conv(kca) + rka / (float)G;
    const float kb = conv(kcb) + rkb / (float)G;
    float cs = 1.f, sn = 0.f;
    if (p < r / 2) {
      double sd, cd;
      sincos((double)(L0 + tt) * inv_freq, &sd, &cd);
      cs = (float)cd;
      sn = (float)sd;
    }
    T* ob = outs + (wave * tpw + sub) * (G + 2) * d;
    // squared lengths of the G query heads and the key head, reduced together
    float ss[G + 1];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) ss[hh] = qa[hh] * qa[hh] + qb[hh] * qb[hh];
    ss[G] = ka * ka + kb * kb;
#pragma unroll
    for (int o = spt / 2; o > 0; o >>= 1)
#pragma unroll
      for (int i = 0; i <= G; ++i) ss[i] += __shfl_xor(ss[i], o, 64);
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float sc = sqrt_d / fmaxf(sqrtf(ss[hh]), 1e-12f);
      float va = qa[hh] * sc, vb = qb[hh] * sc;
      if (p < r / 2) {
        const float ra = va * cs - vb * sn, rb = vb * cs + va * sn;
        va = ra;
        vb = rb;
      }
      ob[hh * d + da] = Act<T>::cvt(va);
      ob[hh * d + db] = Act<T>::cvt(vb);
    }
    {
      const float sc = temp * sqrt_d / fmaxf(sqrtf(ss[G]), 1e-12f);
      float va = ka * sc, vb = kb * sc;
      if (p < r / 2) {
        const float ra = va * cs - vb * sn, rb = vb * cs + va * sn;
        va = ra;
        vb = rb;
      }
      // values: current half of token t, delayed half of token t - 1
      auto vval = [&](int x) -> T { return x < d / 2 ? x0[GC + x] : x1[GC + x]; };
      const T vda = vval(da), vdb = vval(db);
      ob[G * d + da] = Act<T>::cvt(va);
      ob[G * d + db] = Act<T>::cvt(vb);
      ob[(G + 1) * d + da] = vda;
      ob[(G + 1) * d + db] = vdb;
    }
    // copy the step's rows out in 16-byte chunks (the wave's own LDS rows: LDS
    // operations of one wave complete in order, so no barrier is needed)
    __builtin_amdgcn_wave_barrier();
    {
      const int cpr = d / E16;             // chunks per row
      const int cps = (G + 2) * cpr;       // chunks per token
      for (int i = lane; i < tpw * cps; i += 64) {
        const int sl = i / cps, q = i % cps, rw = q / cpr, ch = q % cpr;
        const int t2 = base + sl;
        if (t2 >= t_end) continue;
        const u32x4 val = *reinterpret_cast<const u32x4*>(outs + ((wave * tpw + sl) * (G + 2) + rw) * d + ch * E16);
        const size_t pos2 = (size_t)(L0 + t2);
        T* dst;
        T* tap;
        if (rw < G) {
          dst = a.Q + (((size_t)b * S + t2) * nh + g * G + rw) * d;
          tap = a.q_tap ? a.q_tap + (((size_t)b * nh + g * G + rw) * S + t2) * d : nullptr;
        } else if (rw == G) {
          dst = a.K + (((size_t)b * nkv + g) * a.cap + pos2) * d;
          tap = a.k_tap ? a.k_tap + (((size_t)b * nkv + g) * S + t2) * d : nullptr;
        } else {
          dst = a.V + (((size_t)b * nkv + g) * a.cap + pos2) * d;
          tap = a.v_tap ? a.v_tap + (((size_t)b * nkv + g) * S + t2) * d : nullptr;
        }
        *reinterpret_cast<u32x4*>(dst + ch * E16) = val;
        if (tap) *reinterpret_cast<u32x4*>(tap + ch * E16) = val;
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // 3. state for the next call. Only tile 0 reads the old conv_state (in step 1, before
  //    the barrier above), so tile 0 also writes the new one: the q/k conv inputs of
  //    tokens S-2 and S-1 (from P; for S == 1 the older slot is the old slot 1, which
  //    this tile holds in LDS). The last token's normed input becomes prev_hs.
  if (tile == 0) {
    for (int c = threadIdx.x; c < GC; c += blockDim.x) {
      const int gc = gchan(c);
      T* cs = a.conv_state + ((size_t)b * a.C + gc) * 2;
      T s0, s1;
      if (t_end == S) {  // one tile: rows S-2 (or the history row) and S-1 are in LDS
        s0 = xs[S * ROWE + c];
        s1 = xs[(S + 1) * ROWE + c];
      } else {
        s0 = a.P[((size_t)b * S + S - 2) * QR + gc];
        s1 = a.P[((size_t)b * S + S - 1) * QR + gc];
      }
      cs[0] = s0;
      cs[1] = s1;
    }
  }
  if (write_prev) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = threadIdx.x + k * (int)blockDim.x;
      if (i < prev_chunks) *reinterpret_cast<u32x4*>(a.prev_hs + (size_t)b * a.H + i * E16) = prev[k];
    }
  }
}

size_t cca_lds_bytes(int d, int G, int act_bytes) {
  const int GC = (G + 1) * d;
  const size_t xs = ((size_t)kCcaRows * (GC + d) * act_bytes + 15) & ~(size_t)15;
  const size_t outs = (size_t)4 * (128 / d) * (G + 2) * d * act_bytes;  // 4 waves x tokens per step
  return xs + (size_t)GC * 4 * sizeof(float) + outs;
}

template <typename T>
hipError_t launch_cca(const CcaArgs<T>& a, hipStream_t s) {
  dim3 grid((a.S + kCcaTokens - 1) / kCcaTokens, a.nkv, a.B);
  const int G = a.nh / a.nkv;
  const size_t lds = cca_lds_bytes(a.d, G, (int)sizeof(T));
#define ZAYA_CCA_CASE(DD, GG)                                                      \
  if (a.d == DD && G == GG) {                                                      \
    hipLaunchKernelGGL((cca_kernel<T, DD, GG>), grid, dim3(256), lds, s, a);        \
    return hipGetLastError();                                                      \
  }
  ZAYA_CCA_CASE(128, 1) ZAYA_CCA_CASE(128, 2) ZAYA_CCA_CASE(128, 4) ZAYA_CCA_CASE(128, 8)
  ZAYA_CCA_CASE(64, 1) ZAYA_CCA_CASE(64, 2) ZAYA_CCA_CASE(64, 4) ZAYA_CCA_CASE(64, 8)
#undef ZAYA_CCA_CASE
  return hipErrorInvalidValue;
}

template hipError_t launch_cca<bf16_t>(const CcaArgs<bf16_t>&, hipStream_t);
template hipError_t launch_cca<float>(const CcaArgs<float>&, hipStream_t);

}  // namespace zaya
