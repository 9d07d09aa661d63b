// Mixture of experts: token buckets, SwiGLU experts, weighted combine and merge.
//
// ("One expert per token, chosen beside a skip class", "Ablating an expert leaves the
// merge's bias" and "The API / support()" — mlp_activation, mlp_neurons,
// expert_outputs, routed_output, mlp_output — on the nnterp page; "Printout":
// ZayaExperts with SiLU; the experts are pre-stacked per the JANGTQ2 card.)
//
//   bucket:  ids = routed tokens grouped by expert, ascending within an expert
//            (stable), offsets = exclusive prefix of the per-expert counts; skip
//            tokens belong to no bucket.
//   gate/up: act = rnd(silu(rnd(x Wg^T))), neurons = rnd(act * rnd(x Wu^T))
//   down:    y = rnd(neurons Wd^T); routed = rnd(w * y)
//            mlp_output = rnd(rnd(routed + hsb) * hss); out = f32(f32(h + rb) * rs) + mlp_output
//
// Grouped GEMMs: the grid is an upper bound on the (expert, column tile, row tile)
// items, (ceil(T/BM) + E) x column tiles; each workgroup walks the E+1 offsets to find
// its item (see moe_item) and exits if it has none, so nothing waits on the host.
// Gate and up weight rows are interleaved in 16-row blocks inside each weight tile,
// so every lane holds a gate and an up accumulator for the same outputs and SwiGLU
// happens in registers.
#include "common.h"
#include "gemm_core.h"
#include "kernels.h"

namespace zaya {

// ----------------------------------------------------------------------------- buckets

// One workgroup of 1024 threads. Tokens are taken in passes of up to kBucketPer
// chunks of 1024 (chunk j: tokens pass0 + 1024 j + tid) whose classes are loaded at
// once and kept in registers (up to 8192 tokens the second sweep reuses them). Counts
// use LDS atomics; placement ranks each token among the same-expert tokens of its wave
// with ballots and adds the counts of the earlier waves, chunk by chunk, so ids stay
// ascending within an expert.
constexpr int kBucketPer = 8;

__global__ __launch_bounds__(1024) void bucket_kernel(const int32_t* __restrict__ cls, int ntok, int E,
                                                      int32_t* __restrict__ offsets, int32_t* __restrict__ ids) {
  __shared__ int cnt[32];
  __shared__ int base[32];
  __shared__ int wcnt[16][32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const unsigned long long lt = (1ull << lane) - 1ull;
  const bool single = ntok <= kBucketPer * 1024;
  int c[kBucketPer];
  auto load = [&](int pass0) {
#pragma unroll
    for (int j = 0; j < kBucketPer; ++j) {
      const int t = pass0 + j * 1024 + tid;
      c[j] = t < ntok ? cls[t] : -1;
    }
  };
  if (tid < 32) cnt[tid] = 0;
  __syncthreads();
  for (int pass0 = 0; pass0 < ntok; pass0 += kBucketPer * 1024) {
    load(pass0);
#pragma unroll
    for (int j = 0; j < kBucketPer; ++j)
      if (c[j] >= 0 && c[j] < E) atomicAdd(&cnt[c[j]], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int e = 0; e < E; ++e) {
      base[e] = run;
      offsets[e] = run;
      run += cnt[e];
    }
    offsets[E] = run;
  }
  __syncthreads();
  for (int pass0 = 0; pass0 < ntok; pass0 += kBucketPer * 1024) {
    if (!single) load(pass0);
    const int nch = min(kBucketPer, (ntok - pass0 + 1023) / 1024);
#pragma unroll
    for (int j = 0; j < kBucketPer; ++j) {
      if (j >= nch) break;
      int rank = 0;
      for (int e = 0; e < E; ++e) {
        const unsigned long long m = __ballot(c[j] == e);
        if (lane == 0) wcnt[wave][e] = __popcll(m);
        if (c[j] == e) rank = __popcll(m & lt);
      }
      __syncthreads();
      if (c[j] >= 0 && c[j] < E) {
        int pos = base[c[j]] + rank;
        for (int w = 0; w < wave; ++w) pos += wcnt[w][c[j]];
        ids[pos] = pass0 + j * 1024 + tid;
      }
      __syncthreads();
      if (tid < E) {
        int add = 0;
        for (int w = 0; w < 16; ++w) add += wcnt[w][tid];
        base[tid] += add;
      }
      __syncthreads();
    }
  }
}

// Up to kBucketPer * 1024 tokens in one sweep: every thread keeps its classes in
// registers; per (chunk, wave, expert) counts come from ballots, one wave per expert
// scans them into that expert's running prefix in (chunk, wave) order, and each token's
// slot is its expert's offset + the prefix of its (chunk, wave) + its rank in the wave.
// Three barriers in all.
__global__ __launch_bounds__(1024) void bucket_small_kernel(const int32_t* __restrict__ cls, int ntok, int E,
                                                            int32_t* __restrict__ offsets, int32_t* __restrict__ ids) {
  __shared__ int wpre[kBucketPer][16][32];  // counts, then exclusive prefixes within an expert
  __shared__ int base[32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const unsigned long long lt = (1ull << lane) - 1ull;
  const int nch = (ntok + 1023) / 1024;
  int c[kBucketPer], rank[kBucketPer];
#pragma unroll
  for (int j = 0; j < kBucketPer; ++j) {
    const int t = j * 1024 + tid;
    c[j] = t < ntok ? cls[max(min(t, ntok - 1), 0)] : -1;
  }
#pragma unroll
  for (int j = 0; j < kBucketPer; ++j) {
    if (j >= nch) break;
    int mine = 0;
    rank[j] = 0;
    for (int e = 0; e < E; ++e) {
      const unsigned long long m = __ballot(c[j] == e);
      if (lane == e) mine = __popcll(m);
      if (c[j] == e) rank[j] = __popcll(m & lt);
    }
    if (lane < E) wpre[j][wave][lane] = mine;
  }
  __syncthreads();
  // wave w scans the (chunk, wave) counts of experts w, w + 16 (two entries per lane)
  for (int e = wave; e < E; e += 16) {
    const int n = nch * 16, k0 = 2 * lane;
    const int v0 = k0 < n ? wpre[k0 >> 4][k0 & 15][e] : 0;
    const int v1 = k0 + 1 < n ? wpre[(k0 + 1) >> 4][(k0 + 1) & 15][e] : 0;
    int incl = v0 + v1;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    const int excl = incl - v0 - v1;
    if (k0 < n) wpre[k0 >> 4][k0 & 15][e] = excl;
    if (k0 + 1 < n) wpre[(k0 + 1) >> 4][(k0 + 1) & 15][e] = excl + v0;
    const int total = __shfl(incl, 63, 64);
    if (lane == 0) base[e] = total;
  }
  __syncthreads();
  if (wave == 0) {  // expert offsets: exclusive scan of the counts
    const int n = lane < E ? base[lane] : 0;
    int incl = n;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    if (lane < E) {
      base[lane] = incl - n;
      offsets[lane] = incl - n;
    }
    if (lane == E - 1) offsets[E] = incl;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kBucketPer; ++j) {
    if (j >= nch) break;
    if (c[j] >= 0 && c[j] < E) ids[base[c[j]] + wpre[j][wave][c[j]] + rank[j]] = j * 1024 + tid;
  }
}

hipError_t launch_bucket(const int32_t* cls, int ntok, int E, int32_t* offsets, int32_t* ids, hipStream_t s) {
  if (ntok <= kBucketPer * 1024 && E <= 32)
    hipLaunchKernelGGL(bucket_small_kernel, dim3(1), dim3(1024), 0, s, cls, ntok, E, offsets, ids);
  else
    hipLaunchKernelGGL(bucket_kernel, dim3(1), dim3(1024), 0, s, cls, ntok, E, offsets, ids);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- grouped GEMMs

// Expert items of 16 rows read each weight tile once: their weight loads may bypass the
// caches (non-temporal).
constexpr bool kStreamFewRows = true;

// Work items of a grouped GEMM are (expert, column tile, row tile), expert by expert,
// then column tile, row tile fastest. They are dealt to the 8 XCDs in contiguous runs
// (workgroup b runs on XCD b % 8), so at any time the workgroups of one XCD work on
// neighbouring items of one expert: they share its token rows and, across row tiles,
// each weight tile through that XCD's L2. Returns false for workgroups past the real
// items (the grid is sized for the worst case on the host).
__device__ __forceinline__ bool moe_item(const int32_t* __restrict__ off, int E, int BM, int ntn, int& e_out,
                                         int& r0_out, int& n_out, int& nt_out) {
  int tiles = 0;
  for (int e = 0; e < E; ++e) tiles += (off[e + 1] - off[e] + BM - 1) / BM;
  const int n_real = tiles * ntn;
  const int per = (n_real + 7) / 8;
  const int k = (int)blockIdx.x / 8;
  if (k >= per) return false;
  int item = (int)(blockIdx.x % 8) * per + k;
  if (item >= n_real) return false;
  for (int e = 0; e < E; ++e) {
    const int n = off[e + 1] - off[e];
    const int mt = (n + BM - 1) / BM;
    if (item < mt * ntn) {
      e_out = e;
      nt_out = item / mt;
      r0_out = (item % mt) * BM;
      n_out = n;
      return true;
    }
    item -= mt * ntn;
  }
  return false;
}

// Grid for a grouped GEMM: an upper bound on the items, rounded to the 8 XCDs.
static inline int moe_grid(int ntok, int E, int BM, int ntn) {
  const int nmax = ((ntok + BM - 1) / BM + E) * ntn;
  return 8 * ((nmax + 7) / 8);
}

// BN weight rows per item = BN/2 activation columns, gate and up in alternating 16-row
// blocks.
template <typename T, int BM, int WM, int WN, int BN = 128>
__global__ __launch_bounds__(WM* WN * 64)
__attribute__((amdgpu_waves_per_eu(GemmTile<T, BM, BN, WM, WN>::kWavesPerEU))) void moe_gateup_kernel(MoeArgs<T> a) {
  constexpr int CN = BN / 2;  // activation columns per item
  using Tile = GemmTile<T, BM, BN, WM, WN, (BM <= 16 && kStreamFewRows)>;  // 16-row items: one item per weight tile
  static_assert(Tile::kTN % 2 == 0, "each wave needs gate/up pairs");
  __shared__ __attribute__((aligned(16))) char smem[Tile::kLdsBytes];
  int e, r0, n_e, j;  // j: activation columns [CN j, CN j + CN)
  if (!moe_item(a.offsets, a.E, BM, a.I / CN, e, r0, n_e, j)) return;
  const int base = a.offsets[e] + r0;
  const int rows = min(BM, n_e - r0);
  Tile t;
  t.set_a([&](int r) -> const T* { return a.hn + (size_t)a.ids[base + min(r, rows - 1)] * a.H; });
  const T* Wg = a.W_gu + (size_t)e * 2 * a.I * a.H;
  t.set_b([&](int r) -> const T* {
    const int blk = r >> 4, w16 = r & 15;
    const int row = ((blk & 1) ? a.I : 0) + CN * j + (blk >> 1) * 16 + w16;
    return Wg + (size_t)row * a.H;
  });
  t.run(smem, a.H / Tile::kBK);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
#pragma unroll
  for (int i = 0; i < Tile::kTM; ++i) {
    const int m = wm * Tile::kTM * 16 + i * 16 + (lane & 15);
    if (m >= rows) continue;
    T* nrow = a.neurons + (size_t)(base + m) * a.I;
#pragma unroll
    for (int pp = 0; pp < Tile::kTN / 2; ++pp) {
      const int col = CN * j + (wn * (Tile::kTN / 2) + pp) * 16 + (lane >> 4) * 4;
      float v[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float gt = Act<T>::rnd(t.acc[i][2 * pp][c]);
        const float ut = Act<T>::rnd(t.acc[i][2 * pp + 1][c]);
        const float act = Act<T>::rnd(gt / (1.0f + expf(-gt)));
        v[c] = Act<T>::rnd(act * ut);
      }
      store4(nrow + col, v);
    }
  }
}

template <typename T, int BM, int WM, int WN, int BN = 128>
__global__ __launch_bounds__(WM* WN * 64)
__attribute__((amdgpu_waves_per_eu(GemmTile<T, BM, BN, WM, WN>::kWavesPerEU))) void moe_down_kernel(MoeArgs<T> a) {
  using Tile = GemmTile<T, BM, BN, WM, WN, (BM <= 16 && kStreamFewRows)>;  // 16-row items: one item per weight tile
  __shared__ __attribute__((aligned(16))) char smem[Tile::kLdsBytes];
  int e, r0, n_e, c;
  if (!moe_item(a.offsets, a.E, BM, a.H / BN, e, r0, n_e, c)) return;
  const int n0 = c * BN;
  const int base = a.offsets[e] + r0;
  const int rows = min(BM, n_e - r0);
  Tile t;
  t.set_a([&](int r) -> const T* { return a.neurons + (size_t)(base + min(r, rows - 1)) * a.I; });
  const T* Wd = a.W_dn + (size_t)e * a.H * a.I;
  t.set_b([&](int r) -> const T* { return Wd + (size_t)(n0 + r) * a.I; });
  t.run(smem, a.I / Tile::kBK);
  t.epilogue([&](int m, int nl, const float* v) {
    if (m >= rows) return;
    const int tok = a.ids[base + m];
    const int n = n0 + nl;
    const float w = Act<T>::tof(a.wts[tok]);
    float hv[4], b1[4], s1[4], b2[4], s2[4], ro[4], mo[4], o[4];
    load4(a.h + (size_t)tok * a.H + n, hv);
    load4(a.hsb + n, b1);
    load4(a.hss + n, s1);
    load4(a.rb + n, b2);
    load4(a.rs + n, s2);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float y = Act<T>::rnd(v[c]);
      ro[c] = Act<T>::rnd(w * y);
      mo[c] = Act<T>::rnd(Act<T>::rnd(ro[c] + b1[c]) * s1[c]);
      o[c] = fadd(fmul(fadd(hv[c], b2[c]), s2[c]), mo[c]);
    }
    store4(a.out + (size_t)tok * a.H + n, o);
    if (a.routed_tap) store4(a.routed_tap + (size_t)tok * a.H + n, ro);
    if (a.mlp_tap) store4(a.mlp_tap + (size_t)tok * a.H + n, mo);
  });
}

template <typename T, int BM, int WM, int WN, int BN = 128>
static hipError_t launch_gateup_cfg(const MoeArgs<T>& a, hipStream_t s) {
  hipLaunchKernelGGL((moe_gateup_kernel<T, BM, WM, WN, BN>), dim3(moe_grid(a.ntok, a.E, BM, a.I / (BN / 2))),
                     dim3(WM * WN * 64), 0, s, a);
  return hipGetLastError();
}

template <typename T, int BM, int WM, int WN, int BN = 128>
static hipError_t launch_down_cfg(const MoeArgs<T>& a, hipStream_t s) {
  hipLaunchKernelGGL((moe_down_kernel<T, BM, WM, WN, BN>), dim3(moe_grid(a.ntok, a.E, BM, a.H / BN)),
                     dim3(WM * WN * 64), 0, s, a);
  return hipGetLastError();
}

// Row tile by load: 16-row tiles when experts see only a few tokens each (decode), with
// 64 output columns per item for down so its items (about twice the CU count) fill the
// chip; otherwise 128 x 128 tiles.
template <typename T>
hipError_t launch_moe_gateup(const MoeArgs<T>& a, hipStream_t s) {
  if (a.ntok <= 0) return hipSuccess;
  if (a.ntok <= 32 * a.E) return launch_gateup_cfg<T, 16, 1, 4>(a, s);
  return launch_gateup_cfg<T, 128, 2, 2>(a, s);
}

template <typename T>
hipError_t launch_moe_down(const MoeArgs<T>& a, hipStream_t s) {
  if (a.ntok <= 0) return hipSuccess;
  if (a.ntok <= 32 * a.E) return launch_down_cfg<T, 16, 1, 4, 64>(a, s);
  return launch_down_cfg<T, 128, 2, 2>(a, s);
}

// ----------------------------------------------------------------------------- FP8 experts
//
// Expert weights stored as OCP FP8 E4M3 bytes with one fp32 scale per weight row
// (weight = byte value x scale); activations bf16. A workgroup takes one item =
// (expert, tile of up to 16 of its tokens, 64 output rows): the token rows are staged
// once in LDS (whole K, rows padded by 16 bytes so the fragment reads of 16 rows hit
// distinct banks), and each wave streams its 16 weight rows (gate/up: 16 gate and the
// matching 16 up rows) straight from memory into registers, 16 bytes per lane per 64
// K elements, eight such loads ahead of the MFMAs. The bytes are widened to bf16 in
// registers (exactly: every E4M3 value is a bf16 value) and fed to the bf16 MFMA; the
// row scale multiplies the fp32 sum before the rounding the bf16 path applies. K is
// visited in a fixed order per lane group (elements 64 s + 16 grp .. + 16 for both
// operands), which only permutes the terms of each dot product.
constexpr int kF8Tok = 16;
constexpr int kF8Ahead = 8;
constexpr bool kF8Stream = false;  // non-temporal weight loads measured slower for FP8 items (decode gate/up 40 vs 31 us)

__device__ __forceinline__ void f8x16_to_bf16(const u32x4 q, bf16x8_t& lo, bf16x8_t& hi) {
  u32x4 a, b;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const f32x2_t p0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[k], false);
    const f32x2_t p1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[k], true);
    a[2 * k] = pack_bf16x2(p0.x, p0.y);
    a[2 * k + 1] = pack_bf16x2(p1.x, p1.y);
    const f32x2_t r0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[k + 2], false);
    const f32x2_t r1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[k + 2], true);
    b[2 * k] = pack_bf16x2(r0.x, r0.y);
    b[2 * k + 1] = pack_bf16x2(r1.x, r1.y);
  }
  lo = __builtin_bit_cast(bf16x8_t, a);
  hi = __builtin_bit_cast(bf16x8_t, b);
}

// STREAM: every weight tile is read by one item (few tokens per expert): non-temporal
// weight loads.
template <bool GATEUP, bool STREAM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void moe_f8_kernel(MoeArgs<bf16_t> a) {
  extern __shared__ __attribute__((aligned(16))) char xs[];  // kF8Tok rows x (K bf16 + 16 bytes)
  const int K = GATEUP ? a.H : a.I;
  const int ntn = (GATEUP ? a.I : a.H) / 64;
  int e, r0, n_e, j;
  if (!moe_item(a.offsets, a.E, kF8Tok, ntn, e, r0, n_e, j)) return;
  const int base = a.offsets[e] + r0;
  const int rows = min(kF8Tok, n_e - r0);
  const int pitch = K * 2 + 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, grp = lane >> 4;

  // weight rows of this lane (byte pointers at its 16-byte column) and the first loads
  const uint8_t* W = reinterpret_cast<const uint8_t*>(GATEUP ? (const void*)a.W_gu : (const void*)a.W_dn) +
                     (size_t)e * (GATEUP ? 2 * (size_t)a.I * a.H : (size_t)a.H * a.I);
  const int n_row = 64 * j + 16 * wave + r16;  // gate row (gate/up) or output row (down)
  const uint8_t* w0 = W + (size_t)n_row * K + grp * 16;
  const uint8_t* w1 = W + (size_t)(GATEUP ? a.I + n_row : n_row) * K + grp * 16;
  const int nds = K / 64;
  auto wload = [](const uint8_t* p) -> u32x4 {
    if constexpr (STREAM) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    else return *reinterpret_cast<const u32x4*>(p);
  };
  u32x4 q0[kF8Ahead], q1[kF8Ahead];
#pragma unroll
  for (int p = 0; p < kF8Ahead; ++p) {
    const int s = min(p, nds - 1);
    q0[p] = wload(w0 + (size_t)s * 64);
    if (GATEUP) q1[p] = wload(w1 + (size_t)s * 64);
  }

  // stage the token rows (rows past the tile repeat its last row; never stored)
  {
    const int cpr = K / 8;  // 16-byte chunks per row
    for (int c0 = threadIdx.x; c0 < kF8Tok * cpr; c0 += 256 * 4) {
      u32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int ch = c0 + u * 256;
        if (ch < kF8Tok * cpr) {
          const int r = ch / cpr, cc = ch % cpr;
          const int rr = min(r, rows - 1);
          const bf16_t* src = GATEUP ? a.hn + (size_t)a.ids[base + rr] * a.H : a.neurons + (size_t)(base + rr) * a.I;
          v[u] = *reinterpret_cast<const u32x4*>(src + cc * 8);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int ch = c0 + u * 256;
        if (ch < kF8Tok * cpr) *reinterpret_cast<u32x4*>(xs + (ch / cpr) * pitch + (ch % cpr) * 16) = v[u];
      }
    }
  }
  __syncthreads();

  const char* xrow = xs + r16 * pitch + grp * 32;
  f32x4 acc0 = f32x4{0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
  for (int s0 = 0; s0 < nds; s0 += kF8Ahead) {
#pragma unroll
    for (int p = 0; p < kF8Ahead; ++p) {
      const int s = s0 + p;
      if (s < nds) {
        const bf16x8_t xa = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4*>(xrow + (size_t)s * 128));
        const bf16x8_t xb = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4*>(xrow + (size_t)s * 128 + 16));
        bf16x8_t wa, wb;
        f8x16_to_bf16(q0[p], wa, wb);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, xa, acc0, 0, 0, 0);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb, xb, acc0, 0, 0, 0);
        if (GATEUP) {
          f8x16_to_bf16(q1[p], wa, wb);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, xa, acc1, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb, xb, acc1, 0, 0, 0);
        }
        // refill this slot kF8Ahead steps ahead (past the end: the last step again)
        const int sn = min(s + kF8Ahead, nds - 1);
        q0[p] = wload(w0 + (size_t)sn * 64);
        if (GATEUP) q1[p] = wload(w1 + (size_t)sn * 64);
      }
    }
  }

  // lane holds rows n = 16 wave + 4 grp + i of the item's 64, for token r16
  if (r16 >= rows) return;
  const int n0 = 64 * j + 16 * wave + 4 * grp;
  if (GATEUP) {
    float sg[4], su[4], v[4];
    load4(a.gu_scale + (size_t)e * 2 * a.I + n0, sg);
    load4(a.gu_scale + (size_t)e * 2 * a.I + a.I + n0, su);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float gt = Act<bf16_t>::rnd(acc0[i] * sg[i]);
      const float ut = Act<bf16_t>::rnd(acc1[i] * su[i]);
      const float act = Act<bf16_t>::rnd(gt / (1.0f + expf(-gt)));
      v[i] = Act<bf16_t>::rnd(act * ut);
    }
    store4(a.neurons + (size_t)(base + r16) * a.I + n0, v);
  } else {
    const int tok = a.ids[base + r16];
    const float wt = Act<bf16_t>::tof(a.wts[tok]);
    float sd[4], hv[4], b1[4], s1[4], b2[4], s2[4], ro[4], mo[4], o[4];
    load4(a.dn_scale + (size_t)e * a.H + n0, sd);
    load4(a.h + (size_t)tok * a.H + n0, hv);
    load4(a.hsb + n0, b1);
    load4(a.hss + n0, s1);
    load4(a.rb + n0, b2);
    load4(a.rs + n0, s2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float y = Act<bf16_t>::rnd(acc0[i] * sd[i]);
      ro[i] = Act<bf16_t>::rnd(wt * y);
      mo[i] = Act<bf16_t>::rnd(Act<bf16_t>::rnd(ro[i] + b1[i]) * s1[i]);
      o[i] = fadd(fmul(fadd(hv[i], b2[i]), s2[i]), mo[i]);
    }
    store4(a.out + (size_t)tok * a.H + n0, o);
    if (a.routed_tap) store4(a.routed_tap + (size_t)tok * a.H + n0, ro);
    if (a.mlp_tap) store4(a.mlp_tap + (size_t)tok * a.H + n0, mo);
  }
}

template <bool GATEUP>
static hipError_t launch_f8(const MoeArgs<bf16_t>& a, hipStream_t s) {
  if (a.ntok <= 0) return hipSuccess;
  const int K = GATEUP ? a.H : a.I;
  const size_t lds = (size_t)kF8Tok * (K * 2 + 16);
  static const hipError_t attr = hipFuncSetAttribute((const void*)moe_f8_kernel<GATEUP, false>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  static const hipError_t attr_s = hipFuncSetAttribute((const void*)moe_f8_kernel<GATEUP, true>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (attr != hipSuccess) return attr;
  if (attr_s != hipSuccess) return attr_s;
  const dim3 grid(moe_grid(a.ntok, a.E, kF8Tok, (GATEUP ? a.I : a.H) / 64));
  if (a.ntok <= kF8Tok * a.E && kF8Stream)  // about one token tile per expert: weights streamed once
    hipLaunchKernelGGL((moe_f8_kernel<GATEUP, true>), grid, dim3(256), lds, s, a);
  else
    hipLaunchKernelGGL((moe_f8_kernel<GATEUP, false>), grid, dim3(256), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_moe_gateup_f8(const MoeArgs<bf16_t>& a, hipStream_t s) { return launch_f8<true>(a, s); }
hipError_t launch_moe_down_f8(const MoeArgs<bf16_t>& a, hipStream_t s) { return launch_f8<false>(a, s); }

template hipError_t launch_moe_gateup<bf16_t>(const MoeArgs<bf16_t>&, hipStream_t);
template hipError_t launch_moe_gateup<float>(const MoeArgs<float>&, hipStream_t);
template hipError_t launch_moe_down<bf16_t>(const MoeArgs<bf16_t>&, hipStream_t);
template hipError_t launch_moe_down<float>(const MoeArgs<float>&, hipStream_t);

}  // namespace zaya
