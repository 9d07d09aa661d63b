// MFMA tile engine for C[m, n] = sum_k A[m, k] * B[n, k] (both operands K-contiguous).
//
// A workgroup of WM x WN waves computes a BM x BN tile; each wave a (BM/WM) x (BN/WN)
// sub-tile made of 16x16 MFMA blocks. Tiles of 128-byte K-slices (64 bf16 or 32 fp32)
// are staged through LDS, double-buffered with register prefetch: the global loads of
// slice k+1 are in flight while slice k feeds the MFMAs. Rows are padded by 16 bytes
// in LDS so the 16-byte fragment reads of 16 consecutive rows spread over the banks.
//
// Operands are swapped on purpose: the MFMA's first operand takes rows of B (the
// weights, index n) and its second rows of A (index m), so each lane ends up holding
// four consecutive n of one m — epilogues then issue 8-/16-byte vector stores.
//
// Row sources are given per 16-byte load chunk as byte pointers (NULL = zero row), so
// the same engine serves dense GEMMs, gathered rows (token buckets) and interleaved
// weight rows (gate/up pairs).
#pragma once
#include "common.h"

namespace zaya {

template <typename T, int BM, int BN, int WM, int WN>
struct GemmTile {
  using MF = Mfma<T>;
  using frag = typename MF::frag;
  static constexpr int kThreads = WM * WN * 64;
  static constexpr int kRowBytes = 128;                    // one K slice of a row
  static constexpr int kLdsRow = kRowBytes + 16;           // padded LDS row stride
  static constexpr int kBK = kRowBytes / (int)sizeof(T);   // K elements per slice
  static constexpr int kKSteps = kBK / 32;                 // MFMA k-steps per slice
  static constexpr int kTM = BM / (WM * 16);
  static constexpr int kTN = BN / (WN * 16);
  static constexpr int kAChunks = (BM * 8 + kThreads - 1) / kThreads;
  static constexpr int kBChunks = (BN * 8 + kThreads - 1) / kThreads;
  static constexpr int kBufBytes = (BM + BN) * kLdsRow;
  static constexpr int kLdsBytes = 2 * kBufBytes;
  static_assert(BM % (WM * 16) == 0 && BN % (WN * 16) == 0, "tile must split into 16x16 blocks");
  static_assert(kKSteps >= 1, "slice too short");

  f32x4 acc[kTM][kTN];
  const char* pa[kAChunks];
  const char* pb[kBChunks];

  __device__ __forceinline__ void zero_acc() {
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Chunk c of the A tile covers row c / 8, bytes (c % 8) * 16 .. +16 of each K slice.
  __device__ __forceinline__ static int chunk_row(int i) { return (int)(threadIdx.x + i * kThreads) >> 3; }
  __device__ __forceinline__ static int chunk_col(int i) { return ((int)(threadIdx.x + i * kThreads) & 7) * 16; }

  // set_a(rowptr): rowptr(r) -> const T* to row r at k = 0 (or NULL for a zero row)
  template <class F>
  __device__ __forceinline__ void set_a(F rowptr) {
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) {
      int r = chunk_row(i);
      const T* p = (r < BM) ? rowptr(r) : nullptr;
      pa[i] = p ? reinterpret_cast<const char*>(p) + chunk_col(i) : nullptr;
    }
  }
  template <class F>
  __device__ __forceinline__ void set_b(F rowptr) {
#pragma unroll
    for (int i = 0; i < kBChunks; ++i) {
      int r = chunk_row(i);
      const T* p = (r < BN) ? rowptr(r) : nullptr;
      pb[i] = p ? reinterpret_cast<const char*>(p) + chunk_col(i) : nullptr;
    }
  }

  __device__ __forceinline__ void load_slice(int kt, uint4* ra, uint4* rb) const {
    const size_t off = (size_t)kt * kRowBytes;
#pragma unroll
    for (int i = 0; i < kAChunks; ++i)
      ra[i] = pa[i] ? *reinterpret_cast<const uint4*>(pa[i] + off) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < kBChunks; ++i)
      rb[i] = pb[i] ? *reinterpret_cast<const uint4*>(pb[i] + off) : make_uint4(0, 0, 0, 0);
  }

  __device__ __forceinline__ static void store_slice(char* buf, const uint4* ra, const uint4* rb) {
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) {
      int r = chunk_row(i);
      if (r < BM) *reinterpret_cast<uint4*>(buf + r * kLdsRow + chunk_col(i)) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < kBChunks; ++i) {
      int r = chunk_row(i);
      if (r < BN) *reinterpret_cast<uint4*>(buf + (BM + r) * kLdsRow + chunk_col(i)) = rb[i];
    }
  }

  __device__ __forceinline__ void compute_slice(const char* buf) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int r16 = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      const int koff = ks * 32 * (int)sizeof(T) + grp * 8 * (int)sizeof(T);
      frag xa[kTM], wb[kTN];
#pragma unroll
      for (int i = 0; i < kTM; ++i)
        xa[i] = MF::load(reinterpret_cast<const T*>(buf + (wm * kTM * 16 + i * 16 + r16) * kLdsRow + koff));
#pragma unroll
      for (int j = 0; j < kTN; ++j)
        wb[j] = MF::load(reinterpret_cast<const T*>(buf + (BM + wn * kTN * 16 + j * 16 + r16) * kLdsRow + koff));
#pragma unroll
      for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j) acc[i][j] = MF::mma(wb[j], xa[i], acc[i][j]);
    }
  }

  // Full K loop over nk slices. lds: kLdsBytes of shared memory.
  __device__ __forceinline__ void run(char* lds, int nk) {
    zero_acc();
    uint4 ra[kAChunks], rb[kBChunks];
    load_slice(0, ra, rb);
    store_slice(lds, ra, rb);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const bool more = kt + 1 < nk;
      if (more) load_slice(kt + 1, ra, rb);
      compute_slice(lds + (kt & 1) * kBufBytes);
      if (more) store_slice(lds + ((kt + 1) & 1) * kBufBytes, ra, rb);
      __syncthreads();
    }
  }

  // Calls f(m_local, n_local, v[4]) for every 4-column group this lane holds;
  // n_local is the first of the four consecutive columns.
  template <class F>
  __device__ __forceinline__ void epilogue(F f) const {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / WN, wn = wave % WN;
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j) {
        const int m = wm * kTM * 16 + i * 16 + (lane & 15);
        const int n = wn * kTN * 16 + j * 16 + (lane >> 4) * 4;
        float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
        f(m, n, v);
      }
  }
};

}  // namespace zaya
