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

// Epilogues in the form GemmTile::epilogue_loaded takes (every read issued before the
// first result): Row / Col / Elem hold what is read per row, per 4-column group and per
// (row, group); m and n are global here (the kernel adds the tile origin).
struct EpiNone {};

template <typename T>
struct EpiStore {
  T* C;
  int ldc;
  using Row = EpiNone;
  using Col = EpiNone;
  using Elem = EpiNone;
  __device__ __forceinline__ void load_row(int, Row&) const {}
  __device__ __forceinline__ void load_col(int, Col&) const {}
  __device__ __forceinline__ void load_elem(int, int, const Row&, Elem&) const {}
  __device__ __forceinline__ void apply(int m, int n, const float* v, const Row&, const Col&, const Elem&) const {
    store4(C + (size_t)m * ldc + n, v);
  }
  // split-K reduction pass: one group at a time
  __device__ __forceinline__ void operator()(int m, int n, const float* v) const { store4(C + (size_t)m * ldc + n, v); }
};

template <typename T>
struct EpiMerge {
  const float* x;
  const T *hsb, *hss, *rb, *rs;
  float* h;
  T* a_tap;
  int H;
  using Row = EpiNone;
  struct Col {
    float b1[4], s1[4], b2[4], s2[4];
  };
  struct Elem {
    float xs[4];
  };
  __device__ __forceinline__ void load_row(int, Row&) const {}
  __device__ __forceinline__ void load_col(int n, Col& c) const {
    load4(hsb + n, c.b1);
    load4(hss + n, c.s1);
    load4(rb + n, c.b2);
    load4(rs + n, c.s2);
  }
  __device__ __forceinline__ void load_elem(int m, int n, const Row&, Elem& e) const {
    load4(x + (size_t)m * H + n, e.xs);
  }
  __device__ __forceinline__ void apply(int m, int n, const float* v, const Row&, const Col& c, const Elem& e) const {
    float a[4], o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float oc = Act<T>::rnd(v[q]);
      a[q] = Act<T>::rnd(Act<T>::rnd(oc + c.b1[q]) * c.s1[q]);
      o[q] = fadd(fmul(fadd(e.xs[q], c.b2[q]), c.s2[q]), a[q]);
    }
    store4(h + (size_t)m * H + n, o);
    if (a_tap) store4(a_tap + (size_t)m * H + n, a);
  }
  __device__ __forceinline__ void operator()(int m, int n, const float* v) const {
    Col c;
    Elem e;
    load_col(n, c);
    load_elem(m, n, Row{}, e);
    apply(m, n, v, Row{}, c, e);
  }
};

template <typename T>
struct EpiRouterIn {
  const T* b;
  const T* rss;
  const T* s_in;  // NULL: block-0 semantics
  T* u;
  int R;
  // Where the state loads read: rss and s_in with a carried state, else the bias with a
  // row stride of 0 (read, never used). Set by the launcher, so the loads need no select.
  const T* rss_ld = nullptr;
  const T* st_ld = nullptr;
  int st_stride = 0;
  using Row = EpiNone;
  struct Col {
    float bb[4], sc[4];
  };
  struct Elem {
    float st[4];
  };
  __device__ __forceinline__ void load_row(int, Row&) const {}
  // the state loads are unconditional, so no branch separates them
  __device__ __forceinline__ void load_col(int n, Col& c) const {
    load4(b + n, c.bb);
    load4(rss_ld + n, c.sc);
  }
  __device__ __forceinline__ void load_elem(int m, int n, const Row&, Elem& e) const {
    load4(st_ld + (size_t)m * st_stride + n, e.st);
  }
  __device__ __forceinline__ void apply(int m, int n, const float* v, const Row&, const Col& c, const Elem& e) const {
    float o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      o[q] = Act<T>::rnd(v[q] + c.bb[q]);
      // computed either way and selected (a branch would pull the state loads into it)
      const float with_state = Act<T>::rnd(o[q] + Act<T>::rnd(c.sc[q] * e.st[q]));
      o[q] = s_in ? with_state : o[q];
    }
    store4(u + (size_t)m * R + n, o);
  }
  __device__ __forceinline__ void operator()(int m, int n, const float* v) const {
    Col c;
    Elem e;
    load_col(n, c);
    load_elem(m, n, Row{}, e);
    apply(m, n, v, Row{}, c, e);
  }
};

// Tile-local indices shifted to the tile's origin for an epilogue of global indices.
template <class Epi>
struct EpiAt {
  const Epi& epi;
  int m0, n0;
  using Row = typename Epi::Row;
  using Col = typename Epi::Col;
  using Elem = typename Epi::Elem;
  __device__ __forceinline__ void load_row(int m, Row& r) const { epi.load_row(m0 + m, r); }
  __device__ __forceinline__ void load_col(int n, Col& c) const { epi.load_col(n0 + n, c); }
  __device__ __forceinline__ void load_elem(int m, int n, const Row& r, Elem& e) const {
    epi.load_elem(m0 + m, n0 + n, r, e);
  }
  __device__ __forceinline__ void apply(int m, int n, const float* v, const Row& r, const Col& c, const Elem& e) const {
    epi.apply(m0 + m, n0 + n, v, r, c, e);
  }
};

// Tiles in raster order after the XCD remap: column tiles fastest (the A row band stays
// in cache while B streams), or with m_fast row tiles fastest (B much larger than A:
// each B column band is then read from memory once while the whole of A stays cached,
// e.g. a tied vocabulary head).
template <typename T, int BM, int BN, int WM, int WN, class Epi, int NST>
__global__ __launch_bounds__(WM* WN * 64)
__attribute__((amdgpu_waves_per_eu(GemmTile<T, BM, BN, WM, WN>::kWavesPerEU))) void gemm_nt_kernel(const T* __restrict__ A, int lda, const T* __restrict__ B,
                                                               int ldb, int M, int N, int K, Epi epi, int m_fast) {
  using Tile = GemmTile<T, BM, BN, WM, WN>;
  __shared__ __attribute__((aligned(16))) char smem[Tile::kLdsBytes];
  const int ntn = (N + BN - 1) / BN, ntm = (M + BM - 1) / BM;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int m0 = (m_fast ? wg % ntm : wg / ntn) * BM, n0 = (m_fast ? wg / ntm : wg % ntn) * BN;
  Tile t;
  t.set_a([&](int r) -> const T* { return A + (size_t)min(m0 + r, M - 1) * lda; });
  t.set_b([&](int r) -> const T* { return B + (size_t)min(n0 + r, N - 1) * ldb; });
  t.template run<NST>(smem, K / Tile::kBK);
  t.epilogue_loaded(EpiAt<Epi>{epi, m0, n0}, min(BM, M - m0), min(BN, N - n0));
}

template <typename T, int BM, int BN, int WM, int WN, class Epi, int NST = 3>
static hipError_t launch_cfg(const T* A, int lda, const T* B, int ldb, int M, int N, int K, Epi epi, hipStream_t s) {
  const int g = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int m_fast = (long)N >= 8L * M;  // B at least 8x larger than A
  hipLaunchKernelGGL((gemm_nt_kernel<T, BM, BN, WM, WN, Epi, NST>), dim3(g), dim3(WM * WN * 64), 0, s, A, lda, B, ldb,
                     M, N, K, epi, m_fast);
  return hipGetLastError();
}

// Split-K for GEMMs with few rows (decode): each workgroup reduces one K range of a
// 64 x 64 output tile into fp32 partials; a second pass sums the ranges in a fixed
// order and applies the epilogue, so results do not depend on scheduling. One launch
// may carry two problems with the same K (their tiles one after the other).
template <typename T>
struct SplitProb {
  const T* A;
  int lda;
  const T* B;
  int ldb;
  int M, N;
  float* part;  // [kparts][M][N]
};

template <typename T>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void gemm_splitk_kernel(SplitProb<T> p1,
                                                                                                  SplitProb<T> p2,
                                                                                                  int ntiles1, int K,
                                                                                                  int kparts) {
  using Tile = GemmTile<T, 64, 64, 2, 2>;
  __shared__ __attribute__((aligned(16))) char smem[Tile::kLdsBytes];
  const bool second = (int)blockIdx.x >= ntiles1;
  const SplitProb<T> p = second ? p2 : p1;
  const int tile = second ? (int)blockIdx.x - ntiles1 : (int)blockIdx.x;
  const int M = p.M, N = p.N;
  const int ntn = (N + 63) / 64;
  const int n0 = (tile % ntn) * 64;
  const int m0 = (tile / ntn) * 64;
  const int kp = blockIdx.y;
  const int kslices = K / Tile::kBK;
  const int s0 = kp * kslices / kparts, s1 = (kp + 1) * kslices / kparts;
  const int koff = s0 * Tile::kBK;
  Tile t;
  t.set_a([&](int r) -> const T* { return p.A + (size_t)min(m0 + r, M - 1) * p.lda + koff; });
  t.set_b([&](int r) -> const T* { return p.B + (size_t)min(n0 + r, N - 1) * p.ldb + koff; });
  t.run(smem, s1 - s0);
  float* pp = p.part + (size_t)kp * M * N;
  t.epilogue([&](int m, int n, const float* v) {
    if (m0 + m < M && n0 + n < N) store4(pp + (size_t)(m0 + m) * N + n0 + n, v);
  });
}

template <class Epi>
__global__ __launch_bounds__(256) void gemm_splitk_reduce_kernel(const float* __restrict__ part, int M, int N,
                                                                 int kparts, Epi epi) {
  const int i = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= M * N) return;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  for (int kp = 0; kp < kparts; ++kp) {
    float w[4];
    load4(part + (size_t)kp * M * N + i, w);
#pragma unroll
    for (int c = 0; c < 4; ++c) v[c] += w[c];
  }
  epi(i / N, i % N, v);
}

// The same reduction over two problems in one launch.
template <class Epi1, class Epi2>
__global__ __launch_bounds__(256) void gemm_splitk_reduce2_kernel(const float* __restrict__ part1, int M1, int N1,
                                                                  const float* __restrict__ part2, int M2, int N2,
                                                                  int kparts, Epi1 epi1, Epi2 epi2) {
  int i = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
  const bool second = i >= M1 * N1;
  if (second) i -= M1 * N1;
  const int M = second ? M2 : M1, N = second ? N2 : N1;
  const float* part = second ? part2 : part1;
  if (i >= M * N) return;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  for (int kp = 0; kp < kparts; ++kp) {
    float w[4];
    load4(part + (size_t)kp * M * N + i, w);
#pragma unroll
    for (int c = 0; c < 4; ++c) v[c] += w[c];
  }
  if (second) epi2(i / N, i % N, v);
  else epi1(i / N, i % N, v);
}

// K parts for a split over `ntiles` 64 x 64 tiles holding `elems` outputs, or 1 when the
// GEMM should not be split.
static int splitk_parts(int ntiles, int K, int kBK, size_t elems, size_t part_bytes) {
  int kparts = 1;
  while (ntiles * kparts * 2 <= 512 && (K / kBK) / (kparts * 2) >= 4 && elems * kparts * 2 * sizeof(float) <= part_bytes)
    kparts *= 2;
  return kparts;
}

// Tile choice. GEMMs with few rows (decode) split K into parts reduced by a second
// pass (they stream weights). Otherwise the tile is picked by a cost model: a CU runs
// two 4-wave workgroups (128x96, 128x128) or one 8-wave workgroup (128x192, 128x256) at
// once, so a shape costs (rounds of resident workgroups) x (workgroups per CU) x (tile
// area), the 8-wave shapes at 0.88 of that: they read and stage each A slice once for
// twice the columns (measured on the q/k/v shape: 35.4 vs 40.2 us; o_proj: 27.4 vs
// 29.4 us). Small grids use 64x64 or 32x64 tiles.
template <typename T, class Epi>
static hipError_t launch_any(const T* A, int lda, const T* B, int ldb, int M, int N, int K, Epi epi, float* part,
                             size_t part_bytes, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  constexpr int kBK = 128 / (int)sizeof(T);
  const long t64 = (long)((M + 63) / 64) * ((N + 63) / 64);
  if (M <= 64 && part) {
    const int ntiles = (int)t64;
    const int kparts = splitk_parts(ntiles, K, kBK, (size_t)M * N, part_bytes);
    if (kparts > 1) {
      const SplitProb<T> p{A, lda, B, ldb, M, N, part};
      hipLaunchKernelGGL(gemm_splitk_kernel<T>, dim3(ntiles, kparts), dim3(256), 0, s, p, p, ntiles, K, kparts);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(gemm_splitk_reduce_kernel<Epi>, dim3((M * N / 4 + 255) / 256), dim3(256), 0, s, part, M, N,
                         kparts, epi);
      return hipGetLastError();
    }
  }
  const long mt = (M + 127) / 128;
  const long t128 = mt * ((N + 127) / 128);
  if (t128 >= 240) {
    const long t96 = mt * ((N + 95) / 96), t192 = mt * ((N + 191) / 192), t256 = mt * ((N + 255) / 256);
    const double c96 = (double)((t96 + 511) / 512) * 2 * 96, c128 = (double)((t128 + 511) / 512) * 2 * 128;
    const double c192 = (double)((t192 + 255) / 256) * 192 * 0.88, c256 = (double)((t256 + 255) / 256) * 256 * 0.88;
    const double best = fmin(fmin(c96, c128), fmin(c192, c256));
    if (best == c192) return launch_cfg<T, 128, 192, 2, 4, Epi, 4>(A, lda, B, ldb, M, N, K, epi, s);
    if (best == c256) return launch_cfg<T, 128, 256, 2, 4, Epi, 3>(A, lda, B, ldb, M, N, K, epi, s);
    if (best == c96) return launch_cfg<T, 128, 96, 2, 2>(A, lda, B, ldb, M, N, K, epi, s);
    return launch_cfg<T, 128, 128, 2, 2>(A, lda, B, ldb, M, N, K, epi, s);
  }
  if (t64 >= 120) return launch_cfg<T, 64, 64, 2, 2>(A, lda, B, ldb, M, N, K, epi, s);
  return launch_cfg<T, 32, 64, 1, 4>(A, lda, B, ldb, M, N, K, epi, s);
}

template <typename T>
hipError_t launch_gemm_store(const T* A, int lda, const T* B, int ldb, int M, int N, int K, T* C, int ldc,
                             float* part, size_t part_bytes, hipStream_t s) {
  return launch_any(A, lda, B, ldb, M, N, K, EpiStore<T>{C, ldc}, part, part_bytes, s);
}

template <typename T>
hipError_t launch_gemm_store_pair(const T* A1, int lda1, const T* B1, int ldb1, int M1, int N1, T* C1, int ldc1,
                                  const T* A2, int lda2, const T* B2, int ldb2, int M2, int N2, T* C2, int ldc2, int K,
                                  float* part, size_t part_bytes, hipStream_t s) {
  constexpr int kBK = 128 / (int)sizeof(T);
  const int t1 = ((M1 + 63) / 64) * ((N1 + 63) / 64), t2 = ((M2 + 63) / 64) * ((N2 + 63) / 64);
  const size_t e1 = (size_t)M1 * N1, e2 = (size_t)M2 * N2;
  const int kparts = (M1 <= 64 && M2 <= 64 && part) ? splitk_parts(t1 + t2, K, kBK, e1 + e2, part_bytes) : 1;
  if (kparts == 1) {  // not worth a split: two ordinary launches
    hipError_t e = launch_gemm_store<T>(A1, lda1, B1, ldb1, M1, N1, K, C1, ldc1, part, part_bytes, s);
    if (e != hipSuccess) return e;
    return launch_gemm_store<T>(A2, lda2, B2, ldb2, M2, N2, K, C2, ldc2, part, part_bytes, s);
  }
  const SplitProb<T> p1{A1, lda1, B1, ldb1, M1, N1, part}, p2{A2, lda2, B2, ldb2, M2, N2, part + e1 * kparts};
  hipLaunchKernelGGL(gemm_splitk_kernel<T>, dim3(t1 + t2, kparts), dim3(256), 0, s, p1, p2, t1, K, kparts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gemm_splitk_reduce2_kernel<EpiStore<T>, EpiStore<T>>),
                     dim3((unsigned)((e1 + e2) / 4 + 255) / 256), dim3(256), 0, s, p1.part, M1, N1, p2.part, M2, N2,
                     kparts, EpiStore<T>{C1, ldc1}, EpiStore<T>{C2, ldc2});
  return hipGetLastError();
}

template <typename T>
int launch_gemm_pair_parts(const T* A1, int lda1, const T* B1, int ldb1, int M1, int N1, const T* A2, int lda2,
                           const T* B2, int ldb2, int M2, int N2, int K, float* part, size_t part_bytes, hipStream_t s) {
  constexpr int kBK = 128 / (int)sizeof(T);
  if (M1 > 64 || M2 > 64 || !part) return 0;
  const int t1 = ((M1 + 63) / 64) * ((N1 + 63) / 64), t2 = ((M2 + 63) / 64) * ((N2 + 63) / 64);
  const size_t e1 = (size_t)M1 * N1, e2 = (size_t)M2 * N2;
  const int kparts = splitk_parts(t1 + t2, K, kBK, e1 + e2, part_bytes);
  if (kparts == 1) return 0;
  const SplitProb<T> p1{A1, lda1, B1, ldb1, M1, N1, part}, p2{A2, lda2, B2, ldb2, M2, N2, part + e1 * kparts};
  hipLaunchKernelGGL(gemm_splitk_kernel<T>, dim3(t1 + t2, kparts), dim3(256), 0, s, p1, p2, t1, K, kparts);
  return hipGetLastError() == hipSuccess ? kparts : -1;
}

template <typename T>
int launch_gemm_parts(const T* A, int lda, const T* B, int ldb, int M, int N, int K, float* part, size_t part_bytes,
                      hipStream_t s) {
  constexpr int kBK = 128 / (int)sizeof(T);
  if (M > 64 || !part) return 0;
  const int ntiles = ((M + 63) / 64) * ((N + 63) / 64);
  const int kparts = splitk_parts(ntiles, K, kBK, (size_t)M * N, part_bytes);
  if (kparts == 1) return 0;
  const SplitProb<T> p{A, lda, B, ldb, M, N, part};
  hipLaunchKernelGGL(gemm_splitk_kernel<T>, dim3(ntiles, kparts), dim3(256), 0, s, p, p, ntiles, K, kparts);
  return hipGetLastError() == hipSuccess ? kparts : -1;
}

template <typename T>
hipError_t launch_gemm_merge(const T* O, const T* Wo, int M, int H, int K, const float* x, const T* hsb, const T* hss,
                             const T* rb, const T* rs, float* h, T* a_tap, float* part, size_t part_bytes,
                             hipStream_t s) {
  return launch_any(O, K, Wo, K, M, H, K, EpiMerge<T>{x, hsb, hss, rb, rs, h, a_tap, H}, part, part_bytes, s);
}

template <typename T>
hipError_t launch_gemm_router_in(const T* hn, const T* Wd, int M, int R, int H, const T* b, const T* rss,
                                 const T* s_in, T* u, float* part, size_t part_bytes, hipStream_t s) {
  EpiRouterIn<T> epi{b, rss, s_in, u, R};
  epi.rss_ld = s_in ? rss : b;
  epi.st_ld = s_in ? s_in : b;
  epi.st_stride = s_in ? R : 0;
  return launch_any(hn, H, Wd, H, M, R, H, epi, part, part_bytes, s);
}

#define ZAYA_INST(T)                                                                                                 \
  template hipError_t launch_gemm_store<T>(const T*, int, const T*, int, int, int, int, T*, int, float*, size_t,     \
                                           hipStream_t);                                                             \
  template hipError_t launch_gemm_merge<T>(const T*, const T*, int, int, int, const float*, const T*, const T*,      \
                                           const T*, const T*, float*, T*, float*, size_t, hipStream_t);             \
  template hipError_t launch_gemm_router_in<T>(const T*, const T*, int, int, int, const T*, const T*, const T*, T*, \
                                               float*, size_t, hipStream_t);                                         \
  template hipError_t launch_gemm_store_pair<T>(const T*, int, const T*, int, int, int, T*, int, const T*, int,      \
                                                const T*, int, int, int, T*, int, int, float*, size_t, hipStream_t); \
  template int launch_gemm_parts<T>(const T*, int, const T*, int, int, int, int, float*, size_t, hipStream_t);    \
  template int launch_gemm_pair_parts<T>(const T*, int, const T*, int, int, int, const T*, int, const T*, int, int, \
                                         int, int, float*, size_t, hipStream_t);
ZAYA_INST(bf16_t)
ZAYA_INST(float)
#undef ZAYA_INST

}  // namespace zaya
