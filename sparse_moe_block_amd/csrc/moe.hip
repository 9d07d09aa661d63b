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

hipError_t launch_bucket(const int32_t* cls, int ntok, int E, int32_t* offsets, int32_t* ids, hipStream_t s) {
  hipLaunchKernelGGL(bucket_kernel, dim3(1), dim3(1024), 0, s, cls, ntok, E, offsets, ids);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- grouped GEMMs

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

template <typename T, int BM, int WM, int WN>
__global__ __launch_bounds__(WM* WN * 64)
__attribute__((amdgpu_waves_per_eu(GemmTile<T, BM, 128, WM, WN>::kWavesPerEU))) void moe_gateup_kernel(MoeArgs<T> a) {
  constexpr int BN = 128;  // 64 activation columns: gate and up in alternating 16-row blocks
  using Tile = GemmTile<T, BM, BN, WM, WN>;
  static_assert(Tile::kTN % 2 == 0, "each wave needs gate/up pairs");
  __shared__ __attribute__((aligned(16))) char smem[Tile::kLdsBytes];
  int e, r0, n_e, j;  // j: activation columns [64j, 64j + 64)
  if (!moe_item(a.offsets, a.E, BM, a.I / 64, e, r0, n_e, j)) return;
  const int base = a.offsets[e] + r0;
  const int rows = min(BM, n_e - r0);
  Tile t;
  t.set_a([&](int r) -> const T* { return a.hn + (size_t)a.ids[base + min(r, rows - 1)] * a.H; });
  const T* Wg = a.W_gu + (size_t)e * 2 * a.I * a.H;
  t.set_b([&](int r) -> const T* {
    const int blk = r >> 4, w16 = r & 15;
    const int row = ((blk & 1) ? a.I : 0) + 64 * j + (blk >> 1) * 16 + w16;
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
      const int col = 64 * j + (wn * (Tile::kTN / 2) + pp) * 16 + (lane >> 4) * 4;
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

template <typename T, int BM, int WM, int WN>
__global__ __launch_bounds__(WM* WN * 64)
__attribute__((amdgpu_waves_per_eu(GemmTile<T, BM, 128, WM, WN>::kWavesPerEU))) void moe_down_kernel(MoeArgs<T> a) {
  constexpr int BN = 128;
  using Tile = GemmTile<T, BM, BN, WM, WN>;
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

template <typename T, int BM, int WM, int WN>
static hipError_t launch_gateup_cfg(const MoeArgs<T>& a, hipStream_t s) {
  hipLaunchKernelGGL((moe_gateup_kernel<T, BM, WM, WN>), dim3(moe_grid(a.ntok, a.E, BM, a.I / 64)),
                     dim3(WM * WN * 64), 0, s, a);
  return hipGetLastError();
}

template <typename T, int BM, int WM, int WN>
static hipError_t launch_down_cfg(const MoeArgs<T>& a, hipStream_t s) {
  hipLaunchKernelGGL((moe_down_kernel<T, BM, WM, WN>), dim3(moe_grid(a.ntok, a.E, BM, a.H / 128)),
                     dim3(WM * WN * 64), 0, s, a);
  return hipGetLastError();
}

// Row tile by load: 16-row tiles when experts see only a few tokens each (decode);
// otherwise 128-row tiles for gate/up and 64-row tiles for down (its K is the expert
// width and its column tiles few, so smaller row tiles keep every CU busy).
template <typename T>
hipError_t launch_moe_gateup(const MoeArgs<T>& a, hipStream_t s) {
  if (a.ntok <= 0) return hipSuccess;
  if (a.ntok <= 32 * a.E) return launch_gateup_cfg<T, 16, 1, 4>(a, s);
  return launch_gateup_cfg<T, 128, 2, 2>(a, s);
}

template <typename T>
hipError_t launch_moe_down(const MoeArgs<T>& a, hipStream_t s) {
  if (a.ntok <= 0) return hipSuccess;
  if (a.ntok <= 32 * a.E) return launch_down_cfg<T, 16, 1, 4>(a, s);
  return launch_down_cfg<T, 64, 2, 2>(a, s);
}

template hipError_t launch_moe_gateup<bf16_t>(const MoeArgs<bf16_t>&, hipStream_t);
template hipError_t launch_moe_gateup<float>(const MoeArgs<float>&, hipStream_t);
template hipError_t launch_moe_down<bf16_t>(const MoeArgs<bf16_t>&, hipStream_t);
template hipError_t launch_moe_down<float>(const MoeArgs<float>&, hipStream_t);

}  // namespace zaya
