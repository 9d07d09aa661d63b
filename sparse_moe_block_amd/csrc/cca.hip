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
#include <algorithm>

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
// With the printout's two convolutions (TWO: conv_k == 2) the convolved q/k channels
// come precomputed (conv2_kernel below) and one more buffer follows:
//   y2s[m][0 .. GC)  the two-stage conv output of token t0 + m
// D (head_dim) and GG (query heads per KV head) are compile-time, so the per-head
// loops unroll and the head norms' cross-lane reductions run side by side.
// PARTS: the decode form that sums the projection's split-K partials (a separate
// instantiation, so the prefill form does not carry its registers).
template <typename T, int D, int GG, bool TWO, bool PARTS>
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
  T* y2s = outs + 4 * (128 / d) * (G + 2) * d;
  const int S = a.S, QR = a.qkv_ld;
  const int kcol = nh * d, vccol = nh * d + nkv * d, vdcol = vccol + nkv * d / 2;
  const int L0 = cached_len(a.cache_len, b);
  const bool fresh = L0 == 0;
  const int t0 = tile * kCcaTokens;
  const int t_end = min(S, t0 + kCcaTokens);

  // group channel c -> global channel (column of P, row of conv_w / conv_state)
  auto gchan = [&](int c) { return c < G * d ? g * G * d + c : kcol + g * d + (c - G * d); };

  // the last token's normed input becomes prev_hs (nothing in this kernel reads prev_hs:
  // the delayed value of the token before comes in through vdp)
  constexpr int E16 = 16 / (int)sizeof(T);
  if (t_end == S && g == 0) {
    const int prev_chunks = a.H / E16;
    u32x4 prev[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = threadIdx.x + k * (int)blockDim.x;
      if (i < prev_chunks) prev[k] = *reinterpret_cast<const u32x4*>(a.xn + ((size_t)b * S + S - 1) * a.H + i * E16);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = threadIdx.x + k * (int)blockDim.x;
      if (i < prev_chunks) *reinterpret_cast<u32x4*>(a.prev_hs + (size_t)b * a.H + i * E16) = prev[k];
    }
  }

  // 1. stage projection rows of tokens t0-2 .. t_end-1 (16-byte chunks of the four
  //    contiguous segments), the history rows from conv_state / zeros, and the conv
  //    taps. Each loop issues its loads in batches of kBatch per thread before any of
  //    them is stored, so the tile waits for memory a few times, not once per chunk.
  //    The launch uses 256 threads.
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
    // The conv taps and bias of the group's channels and, for tile 0, the history rows
    // (tokens -2, -1 of a sequence with cached tokens: q/k channels from conv_state) and
    // the delayed value of token -1 (prev_hs @ W_vd^T): requested before the tile rows and
    // held in registers, so all of the tile's loads are in flight together.
    constexpr int kWSlots = ((GG + 1) * D + 255) / 256;      // channels per thread
    constexpr int kHSlots = (2 * (GG + 1) * D + 255) / 256;  // history values per thread
    float wv[kWSlots][4];
#pragma unroll
    for (int k = 0; k < kWSlots; ++k) {
      const int gc = gchan(min((int)threadIdx.x + k * 256, GC - 1));
      if (TWO) {  // depthwise taps (previous, current) and bias: the new state's slot 1
        wv[k][0] = Act<T>::tof(a.conv_w[gc * 2 + 0]);
        wv[k][1] = Act<T>::tof(a.conv_w[gc * 2 + 1]);
        wv[k][2] = Act<T>::tof(a.conv_b[gc]);
        wv[k][3] = 0.f;
      } else {
        wv[k][0] = Act<T>::tof(a.conv_w[gc * 3 + 0]);
        wv[k][1] = Act<T>::tof(a.conv_w[gc * 3 + 1]);
        wv[k][2] = Act<T>::tof(a.conv_w[gc * 3 + 2]);
        wv[k][3] = Act<T>::tof(a.conv_b[gc]);
      }
    }
    T hv[kHSlots];
    float vdv = 0.f;
    if (t0 == 0) {
#pragma unroll
      for (int k = 0; k < kHSlots; ++k) {
        const int i = min((int)threadIdx.x + k * 256, 2 * GC - 1);
        const int rr = i / GC, c = i % GC;
        // kernel 3: rows -2, -1 are slots 0, 1. Two stages: row -1 is slot 0 (the input
        // one token back), used for the new state
        const bool none = fresh || (TWO && rr == 0);
        hv[k] = none ? Act<T>::cvt(0.f) : a.conv_state[((size_t)b * a.C + gchan(c)) * 2 + (TWO ? 0 : rr)];
      }
      if ((int)threadIdx.x < d / 2 && !fresh) {
        const int i = threadIdx.x;
        if (PARTS) {  // the delayed value's split-K partials, summed in ascending order from zero
          const size_t N2 = (size_t)nkv * d / 2, MN2 = (size_t)a.B * N2;
          const float* vp = a.vd_part + b * N2 + g * (d / 2) + i;
          for (int k0 = 0; k0 < a.kparts; k0 += 8) {
            float w8[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) w8[k] = k0 + k < a.kparts ? vp[(k0 + k) * MN2] : 0.f;
#pragma unroll
            for (int k = 0; k < 8; ++k)
              if (k0 + k < a.kparts) vdv += w8[k];
          }
          vdv = Act<T>::tof(Act<T>::cvt(vdv));
        } else {
          vdv = Act<T>::tof(a.vdp[(size_t)b * (nkv * d / 2) + g * (d / 2) + i]);
        }
      }
    }
    if (PARTS) {
      // the projection's split-K partials, summed in ascending order from zero and
      // rounded to T (what the pair's reduction pass would have stored in P)
      const size_t MN = (size_t)a.B * S * QR;
      for (int ch = threadIdx.x; ch < nrows * per_row; ch += nthr) {
        const int rr = ch / per_row, t = t0 - 2 + rr;
        if (t < 0) continue;
        int src, dst;
        chunk_cols(ch % per_row, src, dst);
        const float* pp = a.qkv_part + ((size_t)b * S + t) * QR + src;
        float acc[E16];
#pragma unroll
        for (int q = 0; q < E16; ++q) acc[q] = 0.f;
        for (int k0 = 0; k0 < a.kparts; k0 += 8) {  // eight parts' loads at once, summed in order
          float w[8][E16];
#pragma unroll
          for (int k = 0; k < 8; ++k)
            if (k0 + k < a.kparts)
#pragma unroll
              for (int q = 0; q < E16; q += 4) load4(pp + (k0 + k) * MN + q, &w[k][q]);
#pragma unroll
          for (int k = 0; k < 8; ++k)
            if (k0 + k < a.kparts)
#pragma unroll
              for (int q = 0; q < E16; ++q) acc[q] += w[k][q];
        }
#pragma unroll
        for (int q = 0; q < E16; q += 4) store4(xs + rr * ROWE + dst + q, acc + q);
      }
    } else
    for (int c0 = threadIdx.x; c0 < nrows * per_row; c0 += kBatch * nthr) {
      u32x4 val[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        // indices clamped into range so no load sits behind a branch (rows before the
        // sequence start are the history, written below; chunks past the tile unused)
        const int ch = min(c0 + k * nthr, nrows * per_row - 1);
        const int rr = ch / per_row, t = max(t0 - 2 + rr, 0);
        int src, dst;
        chunk_cols(ch % per_row, src, dst);
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
    if (TWO) {  // the tile's two-stage conv outputs (q then k channels of the group)
      const int per_y = segq + segk;
      const int ny = (t_end - t0) * per_y;
      for (int c0 = threadIdx.x; c0 < ny; c0 += kBatch * nthr) {
        u32x4 val[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          const int ch = min(c0 + k * nthr, ny - 1), cc = ch % per_y;
          const int src = cc < segq ? g * G * d + cc * E16 : kcol + g * d + (cc - segq) * E16;
          val[k] = *reinterpret_cast<const u32x4*>(a.y2 + ((size_t)b * S + t0 + ch / per_y) * a.C + src);
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          const int ch = c0 + k * nthr;
          if (ch < ny) *reinterpret_cast<u32x4*>(y2s + (ch / per_y) * GC + (ch % per_y) * E16) = val[k];
        }
      }
    }
    // the held taps, history rows and delayed value go to LDS
#pragma unroll
    for (int k = 0; k < kWSlots; ++k) {
      const int c = (int)threadIdx.x + k * 256;
      if (c < GC)
#pragma unroll
        for (int q = 0; q < 4; ++q) wsm[c * 4 + q] = wv[k][q];
    }
    if (t0 == 0) {
#pragma unroll
      for (int k = 0; k < kHSlots; ++k) {
        const int i = (int)threadIdx.x + k * 256;
        if (i < 2 * GC) xs[(i / GC) * ROWE + i % GC] = hv[k];
      }
      if ((int)threadIdx.x < d / 2) xs[1 * ROWE + GC + d / 2 + threadIdx.x] = Act<T>::cvt(vdv);
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
  // rotary angle of this lane's token, (L0 + t) inv_freq, as (cos, sin) in fp64: one
  // sincos for the wave's first token, then a rotation by the angle of the 4 tpw tokens
  // between the wave's steps (angle addition; fp64 keeps the drift far below fp32)
  double cd = 1.0, sd = 0.0, cstep = 1.0, sstep = 0.0;
  if (p < r / 2) {
    sincos((double)(L0 + t0 + wave * tpw + sub) * inv_freq, &sd, &cd);
    sincos((double)(4 * tpw) * inv_freq, &sstep, &cstep);
  }
  for (int base = t0 + wave * tpw; base < t_end; base += 4 * tpw) {
    const int t = base + sub;
    const bool active = t < t_end;
    const int tt = active ? t : t_end - 1;
    const int rr = tt - t0 + 2;  // LDS row of token tt
    const T* x0 = xs + rr * ROWE;  // t
    const T* x1 = x0 - ROWE;       // t - 1
    const T* x2 = x1 - ROWE;       // t - 2
    auto conv = [&](int c) -> float {
      if constexpr (TWO) return Act<T>::tof(y2s[(tt - t0) * GC + c]);
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
    const float cs = (float)cd, sn = (float)sd;  // (1, 0) past the rotary dims
    {
      const double c2 = cd * cstep - sd * sstep;
      sd = sd * cstep + cd * sstep;
      cd = c2;
    }
    T* ob = outs + (wave * tpw + sub) * (G + 2) * d;
    // squared lengths of the G query heads and the key head, reduced together
    float ss[G + 1];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) ss[hh] = qa[hh] * qa[hh] + qb[hh] * qb[hh];
    ss[G] = ka * ka + kb * kb;
#pragma unroll
    for (int i = 0; i <= G; ++i) ss[i] = lane_group_sum<spt>(ss[i]);
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
        // a linear cache stores positions below cap only (the host checks cache_len + S
        // <= cap; a replayed call with grown device lengths must not write past it)
        if (rw >= G && !a.ring && L0 + t2 >= a.cap) continue;
        const u32x4 val = *reinterpret_cast<const u32x4*>(outs + ((wave * tpw + sl) * (G + 2) + rw) * d + ch * E16);
        const size_t pos2 = a.ring ? (size_t)((L0 + t2) % a.cap) : (size_t)(L0 + t2);  // cache slot
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
      if (TWO) {  // (input of token S-1, depthwise output of token S-1)
        if (t_end == S) {  // LDS rows S, S+1 are tokens S-2 (the old slot 0 when S = 1), S-1
          const float* w = wsm + c * 4;
          s0 = xs[(S + 1) * ROWE + c];
          s1 = Act<T>::cvt(w[2] + w[0] * Act<T>::tof(xs[S * ROWE + c]) + w[1] * Act<T>::tof(s0));
        } else {
          const float* w = wsm + c * 4;
          s0 = a.P[((size_t)b * S + S - 1) * QR + gc];
          s1 = Act<T>::cvt(w[2] + w[0] * Act<T>::tof(a.P[((size_t)b * S + S - 2) * QR + gc]) +
                           w[1] * Act<T>::tof(s0));
        }
      } else if (t_end == S) {  // one tile: rows S-2 (or the history row) and S-1 are in LDS
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
}

// ---- the two-stage q/k convolution ("Printout": conv_qk_depthwise then conv_qk_grouped)
//
// One workgroup per (64-row tile of the B*S tokens, head h). Thread (chunk, row group)
// reads the inputs of 8 channels of its rows and the two rows before them straight into
// registers and forms, per row, z = [y1(t-1) | y1(t)] (2d values, each depthwise output
// rounded to T; y1(t-1) of one row is y1(t) of the row before it when both are in the
// same sequence). z goes to LDS; y2 = rnd(b2 + W2_h z) is then a [64 x 2d] x [2d x d]
// product on MFMA: wave w takes d/4 output channels, whose weight rows (the first
// operand) it loads once into registers, and all four 16-row blocks of z (the second
// operand) per k-step, so eight accumulations are in flight.
constexpr int kC2Rows = 64;

// Eight act values kept as loaded (16 bytes of bf16, 32 of fp32) and widened on use.
template <typename T> struct Raw8;
template <> struct Raw8<bf16_t> {
  u32x4 w;
  __device__ __forceinline__ void load(const bf16_t* p) { w = *reinterpret_cast<const u32x4*>(p); }
  __device__ __forceinline__ float operator[](int k) const {
    const uint32_t u = w[k >> 1];
    return __uint_as_float((k & 1) ? (u & 0xFFFF0000u) : (u << 16));
  }
};
template <> struct Raw8<float> {
  float4 lo, hi;
  __device__ __forceinline__ void load(const float* p) {
    lo = reinterpret_cast<const float4*>(p)[0];
    hi = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ __forceinline__ float operator[](int k) const {
    const float4& q = k < 4 ? lo : hi;
    switch (k & 3) { case 0: return q.x; case 1: return q.y; case 2: return q.z; default: return q.w; }
  }
};

// Eight floats rounded to the act type (round to nearest even) in their stored form.
template <typename T> struct Pack8;
template <> struct Pack8<bf16_t> {
  u32x4 w;
  __device__ __forceinline__ void set(const float* v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
  }
  __device__ __forceinline__ void zero() { w = u32x4{0u, 0u, 0u, 0u}; }
  __device__ __forceinline__ void store(bf16_t* p) const { *reinterpret_cast<u32x4*>(p) = w; }
};
template <> struct Pack8<float> {
  float4 lo, hi;
  __device__ __forceinline__ void set(const float* v) {
    lo = make_float4(v[0], v[1], v[2], v[3]);
    hi = make_float4(v[4], v[5], v[6], v[7]);
  }
  __device__ __forceinline__ void zero() { lo = hi = make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ __forceinline__ void store(float* p) const {
    reinterpret_cast<float4*>(p)[0] = lo;
    reinterpret_cast<float4*>(p)[1] = hi;
  }
};
// Four floats rounded to the act type and stored (8 bytes of bf16, 16 of fp32).
__device__ __forceinline__ void store4_rne(bf16_t* p, const float* v) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}
__device__ __forceinline__ void store4_rne(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}

template <typename T, int D>
__global__ __launch_bounds__(256) void conv2_kernel(Conv2Args<T> a) {
  extern __shared__ __attribute__((aligned(16))) char c2_lds[];
  constexpr int d = D, K2 = 2 * D;
  constexpr int ZP = K2 + 8;  // z row pitch: the 16 rows of a fragment load start 16 bytes apart
  constexpr int OP = d + 8;   // output tile row pitch, same reason
  constexpr int E16 = 16 / (int)sizeof(T);
  constexpr int CPW = d / 4, NJ = CPW / 16, NKS = K2 / 32;
  constexpr int NCH = d / 8, RG = 256 / NCH, RPG = kC2Rows / RG;  // 8-channel chunks, row groups
  T* z = reinterpret_cast<T*>(c2_lds);  // [kC2Rows][ZP]; later the output tile [kC2Rows][OP]
  using MF = Mfma<T>;
  const int h = blockIdx.y, r0 = blockIdx.x * kC2Rows;
  const int S = a.S, C = a.C, QR = a.qkv_ld, rows = a.B * S;
  const int nrow = min(kC2Rows, rows - r0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, grp = lane >> 4;
  const int ch = threadIdx.x % NCH, rg = threadIdx.x / NCH;
  const int c = ch * 8, m0 = rg * RPG;

  // every load is issued up front, with indices clamped into range (no load behind a
  // branch): this thread's input rows r0+m0-2 .. r0+m0+RPG-1, taps, the cache length
  // of each row's sequence
  Raw8<T> x[RPG + 2];
#pragma unroll
  for (int i = 0; i < RPG + 2; ++i) {
    const int r = min(max(r0 + m0 - 2 + i, 0), rows - 1);
    x[i].load(a.P + (size_t)r * QR + h * d + c);
  }
  Raw8<T> tw[2], b1;  // taps (previous, current) of the 8 channels, interleaved; bias
  tw[0].load(a.conv_w + (size_t)(h * d + c) * 2);
  tw[1].load(a.conv_w + (size_t)(h * d + c) * 2 + 8);
  b1.load(a.conv_b + h * d + c);
  int cl[RPG];
#pragma unroll
  for (int j = 0; j < RPG; ++j) cl[j] = cached_len(a.cache_len, min(r0 + m0 + j, rows - 1) / S);

  // z rows of this thread (rows past the tile are zero)
  Pack8<T> prev, cur;
  auto dw = [&](auto xm1, auto x0, Pack8<T>& y) {  // depthwise output (xm1, x0: k -> value)
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = b1[k] + tw[k >> 2][2 * (k & 3)] * xm1(k) + tw[k >> 2][2 * (k & 3) + 1] * x0(k);
    y.set(v);
  };
  auto row = [&](int i) { return [&x, i](int k) { return x[i][k]; }; };
#pragma unroll
  for (int j = 0; j < RPG; ++j) {
    const int m = m0 + j, r = r0 + m;
    const int t = r - (r / S) * S;
    if (m < nrow) {
      if (t >= 2) {
        if (j == 0) dw(row(j), row(j + 1), prev);
        else prev = cur;  // y1(t-1) = the previous row's y1(t)
        dw(row(j + 1), row(j + 2), cur);
      } else {  // the history comes from the state: slot 0 = input, slot 1 = depthwise output
        Raw8<T> sv[2];
        const bool hist = cl[j] != 0;
        if (hist) {
          const T* st = a.conv_state + ((size_t)(r / S) * C + h * d + c) * 2;
          sv[0].load(st);
          sv[1].load(st + 8);
        }
        auto xm1 = [&](int k) { return hist ? sv[k >> 2][2 * (k & 3)] : 0.f; };
        if (t == 0) {
          float v[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) v[k] = hist ? sv[k >> 2][2 * (k & 3) + 1] : 0.f;
          prev.set(v);  // already act values: exact
          dw(xm1, row(j + 2), cur);
        } else {
          dw(xm1, row(j + 1), prev);
          dw(row(j + 1), row(j + 2), cur);
        }
      }
    } else {
      prev.zero();
      cur.zero();
    }
    prev.store(z + m * ZP + c);
    cur.store(z + m * ZP + d + c);
  }
  // this wave's weight fragments, requested before the barrier (fewer registers live
  // while z is formed; other workgroups on the CU cover the wait)
  typename MF::frag wf[NJ][NKS];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const T* wrow = a.conv2_w + (size_t)(h * d + wave * CPW + j * 16 + r16) * K2 + grp * 8;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) wf[j][ks] = MF::load(wrow + ks * 32);
  }
  __syncthreads();

  f32x4 acc[NJ][kC2Rows / 16];
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int mt = 0; mt < kC2Rows / 16; ++mt) acc[j][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    typename MF::frag zf[kC2Rows / 16];
#pragma unroll
    for (int mt = 0; mt < kC2Rows / 16; ++mt) zf[mt] = MF::load(z + (mt * 16 + r16) * ZP + ks * 32 + grp * 8);
#pragma unroll
    for (int mt = 0; mt < kC2Rows / 16; ++mt)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[j][mt] = MF::mma(wf[j][ks], zf[mt], acc[j][mt]);
  }
  float b2[NJ][4];
#pragma unroll
  for (int j = 0; j < NJ; ++j) load4(a.conv2_b + h * d + wave * CPW + j * 16 + 4 * grp, b2[j]);
  __syncthreads();  // z becomes the output tile
#pragma unroll
  for (int mt = 0; mt < kC2Rows / 16; ++mt)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {  // lane holds channels co .. co+3 of row mt*16 + r16
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = acc[j][mt][i] + b2[j][i];
      store4_rne(z + (mt * 16 + r16) * OP + wave * CPW + j * 16 + 4 * grp, v);
    }
  __syncthreads();
  constexpr int per_row = d / E16;
  for (int q = threadIdx.x; q < nrow * per_row; q += 256) {
    const int m = q / per_row, cc = (q % per_row) * E16;
    *reinterpret_cast<u32x4*>(a.y2 + (size_t)(r0 + m) * C + h * d + cc) =
        *reinterpret_cast<const u32x4*>(z + m * OP + cc);
  }
}

size_t conv2_lds_bytes(int d, int act_bytes) { return (size_t)kC2Rows * (2 * d + 8) * act_bytes; }

// ---- ring caches: the last positions of a fresh prefill, stored at slot p % cap
template <typename T>
__global__ __launch_bounds__(256) void ring_store_kernel(const T* __restrict__ Kw, const T* __restrict__ Vw,
                                                         T* __restrict__ K, T* __restrict__ V, int S, int d,
                                                         int cap, int n) {
  // row i of the (sequence, KV head) pairs' kept positions; chunks of 16 bytes
  constexpr int E16 = 16 / (int)sizeof(T);
  const int cpr = d / E16, keep = min(S, cap), p0 = S - keep;
  const long long total = 2LL * n * keep * cpr;
  for (long long q = (long long)blockIdx.x * 256 + threadIdx.x; q < total; q += (long long)gridDim.x * 256) {
    const int cc = (int)(q % cpr);
    const long long rest = q / cpr;
    const int j = (int)(rest % keep), pair = (int)((rest / keep) % n), kv = (int)(rest / ((long long)keep * n));
    const int p = p0 + j;
    const T* src = (kv ? Vw : Kw) + ((size_t)pair * S + p) * d + cc * E16;
    T* dst = (kv ? V : K) + ((size_t)pair * cap + p % cap) * d + cc * E16;
    *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
  }
}

template <typename T>
hipError_t launch_ring_store(const T* Kw, const T* Vw, T* K, T* V, int B, int nkv, int S, int d, int cap,
                             hipStream_t s) {
  const long long total = 2LL * B * nkv * std::min(S, cap) * (d / (16 / (int)sizeof(T)));
  const int grid = (int)std::min<long long>((total + 255) / 256, 4096);
  hipLaunchKernelGGL((ring_store_kernel<T>), dim3(grid), dim3(256), 0, s, Kw, Vw, K, V, S, d, cap, B * nkv);
  return hipGetLastError();
}
template hipError_t launch_ring_store<bf16_t>(const bf16_t*, const bf16_t*, bf16_t*, bf16_t*, int, int, int, int, int,
                                              hipStream_t);
template hipError_t launch_ring_store<float>(const float*, const float*, float*, float*, int, int, int, int, int,
                                             hipStream_t);

// dynamic LDS the conv2 launches may ask for (fp32, d = 128 needs ~103 KB); the kernel's
// static row tables come on top, within the CU's 160 KB
constexpr int kC2MaxLds = 128 * 1024;

template <typename T>
hipError_t launch_conv2(const Conv2Args<T>& a, hipStream_t s) {
  const int rows = a.B * a.S;
  dim3 grid((rows + kC2Rows - 1) / kC2Rows, a.C / a.d);
  const size_t lds = conv2_lds_bytes(a.d, (int)sizeof(T));
  if (a.d == 128) {
    static const hipError_t attr = hipFuncSetAttribute((const void*)conv2_kernel<T, 128>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kC2MaxLds);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((conv2_kernel<T, 128>), grid, dim3(256), lds, s, a);
  } else if (a.d == 64) {
    static const hipError_t attr = hipFuncSetAttribute((const void*)conv2_kernel<T, 64>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kC2MaxLds);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((conv2_kernel<T, 64>), grid, dim3(256), lds, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template hipError_t launch_conv2<bf16_t>(const Conv2Args<bf16_t>&, hipStream_t);
template hipError_t launch_conv2<float>(const Conv2Args<float>&, hipStream_t);

size_t cca_lds_bytes(int d, int G, int act_bytes, bool two) {
  const int GC = (G + 1) * d;
  const size_t xs = ((size_t)kCcaRows * (GC + d) * act_bytes + 15) & ~(size_t)15;
  const size_t outs = (size_t)4 * (128 / d) * (G + 2) * d * act_bytes;  // 4 waves x tokens per step
  const size_t y2 = two ? (size_t)kCcaTokens * GC * act_bytes : 0;
  return xs + (size_t)GC * 4 * sizeof(float) + outs + y2;
}

template <typename T, int DD, int GG>
static hipError_t launch_cca_dg(const CcaArgs<T>& a, dim3 grid, hipStream_t s) {
  const size_t lds = cca_lds_bytes(DD, GG, (int)sizeof(T), a.conv_k == 2);
  if (a.conv_k == 2) {
    static const hipError_t attr = hipFuncSetAttribute((const void*)cca_kernel<T, DD, GG, true, false>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((cca_kernel<T, DD, GG, true, false>), grid, dim3(256), lds, s, a);
  } else {
    if (a.qkv_part) hipLaunchKernelGGL((cca_kernel<T, DD, GG, false, true>), grid, dim3(256), lds, s, a);
    else hipLaunchKernelGGL((cca_kernel<T, DD, GG, false, false>), grid, dim3(256), lds, s, a);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_cca(const CcaArgs<T>& a, hipStream_t s) {
  // summed partials: the state write of a chunk longer than one tile reads P itself
  if (a.qkv_part && (a.S > kCcaTokens || a.conv_k != 3 || !a.vd_part || a.kparts < 1)) return hipErrorInvalidValue;
  dim3 grid((a.S + kCcaTokens - 1) / kCcaTokens, a.nkv, a.B);
  const int G = a.nh / a.nkv;
#define ZAYA_CCA_CASE(DD, GG) \
  if (a.d == DD && G == GG) return launch_cca_dg<T, DD, GG>(a, grid, s);
  ZAYA_CCA_CASE(128, 1) ZAYA_CCA_CASE(128, 2) ZAYA_CCA_CASE(128, 4) ZAYA_CCA_CASE(128, 8)
  ZAYA_CCA_CASE(64, 1) ZAYA_CCA_CASE(64, 2) ZAYA_CCA_CASE(64, 4) ZAYA_CCA_CASE(64, 8)
#undef ZAYA_CCA_CASE
  return hipErrorInvalidValue;
}

template hipError_t launch_cca<bf16_t>(const CcaArgs<bf16_t>&, hipStream_t);
template hipError_t launch_cca<float>(const CcaArgs<float>&, hipStream_t);

}  // namespace zaya
