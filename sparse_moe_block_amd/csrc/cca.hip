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
// Work split: one workgroup per (16-token tile, KV group, sequence); each wave takes
// one token at a time (two when d = 64). Lane p owns the dim pair (da, db) of every
// head of the group: for p < rope_dim/2 that pair is the rotary pair, so the rotation
// never leaves the lane; the head norms are reductions over the d/2 lanes of a token.
#include "common.h"
#include "kernels.h"

namespace zaya {

constexpr int kCcaTokens = 16;

template <typename T>
__global__ __launch_bounds__(256) void cca_kernel(CcaArgs<T> a) {
  const int b = blockIdx.z, g = blockIdx.y, tile = blockIdx.x;
  const int d = a.d, nh = a.nh, nkv = a.nkv, G = nh / nkv, r = a.rope_dim;
  const int spt = d / 2;          // lanes per token
  const int tpw = 64 / spt;       // tokens per wave step
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane / spt, p = lane % spt;
  const int da = p < r / 2 ? p : r + (p - r / 2);
  const int db = p < r / 2 ? p + r / 2 : r + (d - r) / 2 + (p - r / 2);
  const int L0 = a.cache_len[b];
  const bool fresh = L0 == 0;
  const int S = a.S, QR = a.qkv_ld;
  const int kcol = nh * d, vccol = nh * d + nkv * d, vdcol = vccol + nkv * d / 2;
  const float sqrt_d = sqrtf((float)d);
  const float temp = Act<T>::tof(a.temp[g]);
  // rotary inverse frequency of this lane's pair, in double for large positions
  const double inv_freq = p < r / 2 ? pow((double)a.theta, -2.0 * (double)p / (double)r) : 0.0;

  const int t_begin = tile * kCcaTokens;
  const int t_end = min(S, t_begin + kCcaTokens);
  for (int base = t_begin + wave * tpw; base < t_end; base += 4 * tpw) {
    const int t = base + sub;
    const bool active = t < t_end;
    const int tt = active ? t : t_end - 1;  // inactive half-waves mirror a valid token; results discarded
    const size_t row = (size_t)b * S + tt;
    // gather x(t-2), x(t-1), x(t) for channel c (q or k) at dims da, db
    auto xval = [&](int c, int dt) -> float {
      const int ts = tt - dt;
      if (ts >= 0) return Act<T>::tof(a.P[((size_t)b * S + ts) * QR + c]);
      if (fresh) return 0.f;
      return Act<T>::tof(a.conv_state[((size_t)b * a.C + c) * 2 + (2 + ts)]);  // ts = -2 -> slot 0, -1 -> slot 1
    };
    auto conv = [&](int c) -> float {
      const float w0 = Act<T>::tof(a.conv_w[c * 3 + 0]), w1 = Act<T>::tof(a.conv_w[c * 3 + 1]);
      const float w2 = Act<T>::tof(a.conv_w[c * 3 + 2]);
      return Act<T>::tof(a.conv_b[c]) + w0 * xval(c, 2) + w1 * xval(c, 1) + w2 * xval(c, 0);
    };
    // key head
    const int kca = kcol + g * d + da, kcb = kcol + g * d + db;
    const float pka = Act<T>::tof(a.P[row * QR + kca]), pkb = Act<T>::tof(a.P[row * QR + kcb]);
    float qa[8], qb[8];
    float rka = 0.f, rkb = 0.f;
    for (int hh = 0; hh < G; ++hh) {
      const int h = g * G + hh;
      const int ca = h * d + da, cb = h * d + db;
      const float pqa = Act<T>::tof(a.P[row * QR + ca]), pqb = Act<T>::tof(a.P[row * QR + cb]);
      const float rqa = (pqa + pka) * 0.5f, rqb = (pqb + pkb) * 0.5f;
      rka += rqa;
      rkb += rqb;
      qa[hh] = conv(ca) + rqa;
      qb[hh] = conv(cb) + rqb;
    }
    float ka = conv(kca) + rka / (float)G;
    float kb = conv(kcb) + rkb / (float)G;
    // rotary angle for position L0 + t
    float cs = 1.f, sn = 0.f;
    if (p < r / 2) {
      double ang = (double)(L0 + tt) * inv_freq;
      double sd, cd;
      sincos(ang, &sd, &cd);
      cs = (float)cd;
      sn = (float)sd;
    }
    const size_t pos = (size_t)(L0 + tt);
    // queries
    for (int hh = 0; hh < G; ++hh) {
      const int h = g * G + hh;
      const float ss = group_sum(qa[hh] * qa[hh] + qb[hh] * qb[hh], spt);
      const float sc = sqrt_d / fmaxf(sqrtf(ss), 1e-12f);
      float va = qa[hh] * sc, vb = qb[hh] * sc;
      if (p < r / 2) {
        const float ra = va * cs - vb * sn, rb = vb * cs + va * sn;
        va = ra;
        vb = rb;
      }
      if (active) {
        T* qo = a.Q + (row * nh + h) * d;
        qo[da] = Act<T>::cvt(va);
        qo[db] = Act<T>::cvt(vb);
        if (a.q_tap) {
          T* qt = a.q_tap + (((size_t)b * nh + h) * S + tt) * d;
          qt[da] = Act<T>::cvt(va);
          qt[db] = Act<T>::cvt(vb);
        }
      }
    }
    {
      const float ss = group_sum(ka * ka + kb * kb, spt);
      const float sc = temp * sqrt_d / fmaxf(sqrtf(ss), 1e-12f);
      float va = ka * sc, vb = kb * sc;
      if (p < r / 2) {
        const float ra = va * cs - vb * sn, rb = vb * cs + va * sn;
        va = ra;
        vb = rb;
      }
      // values: current half of token t, delayed half of token t-1
      auto vval = [&](int x) -> float {
        if (x < d / 2) return Act<T>::tof(a.P[row * QR + vccol + g * (d / 2) + x]);
        const int xx = x - d / 2;
        if (tt > 0) return Act<T>::tof(a.P[(row - 1) * QR + vdcol + g * (d / 2) + xx]);
        if (fresh) return 0.f;
        return Act<T>::tof(a.vdp[(size_t)b * (nkv * d / 2) + g * (d / 2) + xx]);
      };
      const float vda = vval(da), vdb = vval(db);
      if (active) {
        T* ko = a.K + (((size_t)b * nkv + g) * a.cap + pos) * d;
        T* vo = a.V + (((size_t)b * nkv + g) * a.cap + pos) * d;
        ko[da] = Act<T>::cvt(va);
        ko[db] = Act<T>::cvt(vb);
        vo[da] = Act<T>::cvt(vda);
        vo[db] = Act<T>::cvt(vdb);
        if (a.k_tap) {
          T* kt = a.k_tap + (((size_t)b * nkv + g) * S + tt) * d;
          kt[da] = Act<T>::cvt(va);
          kt[db] = Act<T>::cvt(vb);
        }
        if (a.v_tap) {
          T* vt = a.v_tap + (((size_t)b * nkv + g) * S + tt) * d;
          vt[da] = Act<T>::cvt(vda);
          vt[db] = Act<T>::cvt(vdb);
        }
      }
    }
  }

  // State for the next call. Only the first tile of a sequence reads the old conv
  // state (tokens 0 and 1), so that tile rewrites it after everyone in it is done.
  if (tile == 0) {
    __syncthreads();
    const int nch = (G + 1) * d;
    for (int i = threadIdx.x; i < nch; i += blockDim.x) {
      const int c = i < G * d ? g * G * d + i : kcol + g * d + (i - G * d);
      T* cs = a.conv_state + ((size_t)b * a.C + c) * 2;
      const T zero = Act<T>::cvt(0.f);
      const T old1 = fresh ? zero : cs[1];
      const T s0 = S >= 2 ? a.P[((size_t)b * S + S - 2) * QR + c] : old1;
      const T s1 = a.P[((size_t)b * S + S - 1) * QR + c];
      cs[0] = s0;
      cs[1] = s1;
    }
  }
  if (tile == gridDim.x - 1 && g == 0) {
    const T* src = a.xn + ((size_t)b * S + S - 1) * a.H;
    T* dst = a.prev_hs + (size_t)b * a.H;
    for (int i = threadIdx.x; i < a.H; i += blockDim.x) dst[i] = src[i];
  }
}

template <typename T>
hipError_t launch_cca(const CcaArgs<T>& a, hipStream_t s) {
  dim3 grid((a.S + kCcaTokens - 1) / kCcaTokens, a.nkv, a.B);
  hipLaunchKernelGGL(cca_kernel<T>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template hipError_t launch_cca<bf16_t>(const CcaArgs<bf16_t>&, hipStream_t);
template hipError_t launch_cca<float>(const CcaArgs<float>&, hipStream_t);

}  // namespace zaya
