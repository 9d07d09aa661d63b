// MFMA tile engine for C[m, n] = sum_k A[m, k] * B[n, k] (both operands K-contiguous).
//
// A workgroup of WM x WN waves computes a BM x BN tile; each wave a (BM/WM) x (BN/WN)
// sub-tile made of 16x16 MFMA blocks. Tiles of 128-byte K-slices (64 bf16 or 32 fp32)
// are staged through a double-buffered LDS tile, fed from a ring of register stages
// that keeps the global loads of the next few slices in flight while one slice feeds
// the MFMAs (a single slice of lookahead leaves every iteration waiting on memory).
// LDS rows are XOR-swizzled (see swz) so fragment reads and slice writes are free of
// bank conflicts without padding.
//
// Operands are swapped on purpose: the MFMA's first operand takes rows of B (the
// weights, index n) and its second rows of A (index m), so each lane ends up holding
// four consecutive n of one m — epilogues then issue 8-/16-byte vector stores.
//
// Row sources are given per 16-byte load chunk as byte pointers, so the same engine
// serves dense GEMMs, gathered rows (token buckets) and interleaved weight rows (gate/up
// pairs).
#pragma once
#include "common.h"

namespace zaya {

// STREAM_B: the B rows are read once per launch (weights of a few-token expert item):
// their loads are non-temporal so they do not evict data that is reused.
template <typename T, int BM, int BN, int WM, int WN, bool STREAM_B = false>
struct GemmTile {
  using MF = Mfma<T>;
  using frag = typename MF::frag;
  static constexpr int kBM = BM, kBN = BN, kWM = WM, kWN = WN;
  static constexpr int kThreads = WM * WN * 64;
  static constexpr int kRowBytes = 128;                    // one K slice of a row
  static constexpr int kBK = kRowBytes / (int)sizeof(T);   // K elements per slice
  static constexpr int kKSteps = kBK / 32;                 // MFMA k-steps per slice
  static constexpr int kTM = BM / (WM * 16);
  static constexpr int kTN = BN / (WN * 16);
  static constexpr int kAChunks = (BM * 8 + kThreads - 1) / kThreads;
  static constexpr int kBChunks = (BN * 8 + kThreads - 1) / kThreads;
  static constexpr int kBufBytes = (BM + BN) * kRowBytes;
  static constexpr int kLdsBytes = 2 * kBufBytes;
  // Waves per SIMD the kernel is compiled for (register budget 512 / waves): 2 for the
  // tiles of 128x96 and up (their LDS already allows only two 4-wave or one 8-wave
  // workgroup per CU), 4 for the smaller ones.
  static constexpr int kWavesPerEU = BM * BN >= 128 * 96 ? 2 : 4;
  static_assert(BM % (WM * 16) == 0 && BN % (WN * 16) == 0, "tile must split into 16x16 blocks");
  static_assert(kKSteps >= 1, "slice too short");

  f32x4 acc[kTM][kTN];
  const char* pa[kAChunks];
  const char* pb[kBChunks];
  // Bytes from one K slice of a B row to the next: one slice (kRowBytes) for row-major
  // operands; a packed operand stores the slices of a row group one after another.
  size_t bstride = kRowBytes;

  // LDS rows are 128 bytes (eight 16-byte chunks) with no padding; chunk j of row r is
  // stored at position j ^ swz(r), swz(r) = (r / 2) % 8. A fragment read has lanes
  // 0-15 on rows 0-15 at chunk c, lanes 16-31 on the same rows at chunk c + 1, and so
  // on; measured on gfx950, a 16-byte LDS read serves 32 lanes at a time over 512
  // bytes of banks, and this mask keeps both halves of such a group on distinct banks
  // (the mask (r % 8) ^ (r / 8 % 2) left 2-way conflicts: 65 vs 120 TB/s of LDS reads).
  // The slice writes (eight lanes per 128-byte row) stay conflict-free.
  __device__ __forceinline__ static int swz(int r) { return (r >> 1) & 7; }
  __device__ __forceinline__ static int lds_off(int r, int chunk) { return r * kRowBytes + ((chunk ^ swz(r)) << 4); }

  __device__ __forceinline__ void zero_acc() {
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Chunk c of the A tile covers row c / 8, bytes (c % 8) * 16 .. +16 of each K slice.
  __device__ __forceinline__ static int chunk_row(int i) { return (int)(threadIdx.x + i * kThreads) >> 3; }
  __device__ __forceinline__ static int chunk_col(int i) { return ((int)(threadIdx.x + i * kThreads) & 7); }

  // set_a(rowptr): rowptr(r) -> const T* to row r at k = 0, for every r < BM. Rows past
  // the problem edge must still point at readable memory (callers clamp them to a
  // valid row); their products land only in outputs the epilogue discards.
  template <class F>
  __device__ __forceinline__ void set_a(F rowptr) {
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) {
      const int r = min(chunk_row(i), BM - 1);
      pa[i] = reinterpret_cast<const char*>(rowptr(r)) + chunk_col(i) * 16;
    }
  }
  template <class F>
  __device__ __forceinline__ void set_b(F rowptr) {
#pragma unroll
    for (int i = 0; i < kBChunks; ++i) {
      const int r = min(chunk_row(i), BN - 1);
      pb[i] = reinterpret_cast<const char*>(rowptr(r)) + chunk_col(i) * 16;
    }
  }

  __device__ __forceinline__ void load_a(int kt, u32x4* ra) const {
    const size_t off = (size_t)kt * kRowBytes;
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) ra[i] = *reinterpret_cast<const u32x4*>(pa[i] + off);
  }
  __device__ __forceinline__ void load_b(int kt, u32x4* rb) const {
    const size_t boff = (size_t)kt * bstride;
#pragma unroll
    for (int i = 0; i < kBChunks; ++i) {
      if constexpr (STREAM_B) rb[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(pb[i] + boff));
      else rb[i] = *reinterpret_cast<const u32x4*>(pb[i] + boff);
    }
  }
  __device__ __forceinline__ void load_slice(int kt, u32x4* ra, u32x4* rb) const {
    load_a(kt, ra);
    load_b(kt, rb);
  }

  __device__ __forceinline__ static void store_slice(char* buf, const u32x4* ra, const u32x4* rb) {
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) {
      const int r = chunk_row(i);
      if ((BM * 8) % kThreads == 0 || r < BM) *reinterpret_cast<u32x4*>(buf + lds_off(r, chunk_col(i))) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < kBChunks; ++i) {
      const int r = chunk_row(i);
      if ((BN * 8) % kThreads == 0 || r < BN)
        *reinterpret_cast<u32x4*>(buf + lds_off(BM + r, chunk_col(i))) = rb[i];
    }
  }

  // Fragment of row r for the 32-wide k-step ks: lane group grp takes elements
  // [8 grp, 8 grp + 8) of the step (16 bytes of bf16, 32 bytes of fp32).
  __device__ __forceinline__ static frag load_frag(const char* buf, int r, int ks, int grp) {
    if constexpr (sizeof(T) == 2) {
      return frag{*reinterpret_cast<const uint4*>(buf + lds_off(r, ks * 4 + grp))};
    } else {
      const int c0 = grp * 2;  // one k-step per slice for fp32
      frag f;
      f.a = *reinterpret_cast<const float4*>(buf + lds_off(r, c0));
      f.b = *reinterpret_cast<const float4*>(buf + lds_off(r, c0 + 1));
      return f;
    }
  }

  __device__ __forceinline__ void compute_slice(const char* buf) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int r16 = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      frag xa[kTM], wb[kTN];
#pragma unroll
      for (int i = 0; i < kTM; ++i) xa[i] = load_frag(buf, wm * kTM * 16 + i * 16 + r16, ks, grp);
#pragma unroll
      for (int j = 0; j < kTN; ++j) wb[j] = load_frag(buf, BM + wn * kTN * 16 + j * 16 + r16, ks, grp);
#pragma unroll
      for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j) acc[i][j] = MF::mma(wb[j], xa[i], acc[i][j]);
    }
  }

  // Full K loop over nk slices. lds: kLdsBytes of shared memory.
  //
  // Global loads run NST (3 or 4) slices ahead of the MFMAs: slice k+1 goes from its
  // register stage to the idle LDS buffer right after slice k's products, and that stage
  // is refilled at once with slice k+NST+1. One barrier per slice. The stages are named
  // variables and the loop is unrolled by hand, so nothing is indexed at run time.
  //
  // The main loop has no data-dependent branches: past the end, the refill re-reads the
  // last slice (never used) and the store fills the idle buffer. Every path then has the
  // same loads in flight, and the compiler waits only for the oldest stage instead of
  // draining all of them before each LDS store.
  struct Stage {
    u32x4 a[kAChunks];
    u32x4 b[kBChunks];
  };
  template <int NST>
  __device__ __forceinline__ void step(char* lds, int kt, int nk, Stage& st) {
    compute_slice(lds + (kt & 1) * kBufBytes);
    store_slice(lds + ((kt + 1) & 1) * kBufBytes, st.a, st.b);
    load_slice(min(kt + NST + 1, nk - 1), st.a, st.b);
    __syncthreads();
  }
  template <int NST = 3>
  __device__ __forceinline__ void run(char* lds, int nk) {
    static_assert(NST == 3 || NST == 4, "three or four register stages");
    if constexpr (NST == 4) {
      run4(lds, nk);
      return;
    }
    zero_acc();
    Stage s0, s1, s2;
    // B rows first: their addresses never wait on a gather (A's rows may be token rows
    // found through the bucket ids)
    load_b(0, s0.b);
    load_b(min(1, nk - 1), s1.b);
    load_b(min(2, nk - 1), s2.b);
    load_a(0, s0.a);
    load_a(min(1, nk - 1), s1.a);
    load_a(min(2, nk - 1), s2.a);
    store_slice(lds, s0.a, s0.b);
    load_slice(min(3, nk - 1), s0.a, s0.b);
    __syncthreads();
    int k0 = 0;
    for (; k0 + 3 <= nk; k0 += 3) {
      step<3>(lds, k0, nk, s1);      // slice k0+1 is in s1
      step<3>(lds, k0 + 1, nk, s2);  // slice k0+2 is in s2
      step<3>(lds, k0 + 2, nk, s0);  // slice k0+3 is in s0
    }
    if (k0 < nk) step<3>(lds, k0, nk, s1);
    if (k0 + 1 < nk) step<3>(lds, k0 + 1, nk, s2);
  }
  __device__ __forceinline__ void run4(char* lds, int nk) {
    zero_acc();
    Stage s0, s1, s2, s3;
    load_b(0, s0.b);
    load_b(min(1, nk - 1), s1.b);
    load_b(min(2, nk - 1), s2.b);
    load_b(min(3, nk - 1), s3.b);
    load_a(0, s0.a);
    load_a(min(1, nk - 1), s1.a);
    load_a(min(2, nk - 1), s2.a);
    load_a(min(3, nk - 1), s3.a);
    store_slice(lds, s0.a, s0.b);
    load_slice(min(4, nk - 1), s0.a, s0.b);
    __syncthreads();
    int k0 = 0;
    for (; k0 + 4 <= nk; k0 += 4) {
      step<4>(lds, k0, nk, s1);
      step<4>(lds, k0 + 1, nk, s2);
      step<4>(lds, k0 + 2, nk, s3);
      step<4>(lds, k0 + 3, nk, s0);
    }
    if (k0 < nk) step<4>(lds, k0, nk, s1);
    if (k0 + 1 < nk) step<4>(lds, k0 + 1, nk, s2);
    if (k0 + 2 < nk) step<4>(lds, k0 + 2, nk, s3);
  }

  // Epilogue with loads: every global read the epilogue needs is issued before the first
  // result is computed (a memory round trip or two per workgroup instead of one per
  // group). Epi provides Row (values per row, loaded first: what the other loads index
  // by), Col (per 4-column group) and Elem (per row and 4-column group) with
  // load_row(m, Row&), load_col(n, Col&), load_elem(m, n, Row, Elem&) and
  // apply(m, n, v[4], Row, Col, Elem); m and n are local to the tile. Rows m >= rows and
  // column groups n >= cols do not exist: they read row 0's / column 0's values and store
  // nothing.
  template <class Epi>
  __device__ __forceinline__ void epilogue_loaded(const Epi& epi, int rows, int cols = BN) const {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / WN, wn = wave % WN;
    typename Epi::Row row[kTM];
    typename Epi::Col col[kTN];
    typename Epi::Elem el[kTM][kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      const int m = wm * kTM * 16 + i * 16 + (lane & 15);
      epi.load_row(m < rows ? m : 0, row[i]);
    }
#pragma unroll
    for (int j = 0; j < kTN; ++j) {
      const int n = wn * kTN * 16 + j * 16 + (lane >> 4) * 4;
      epi.load_col(n < cols ? n : 0, col[j]);
    }
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      const int m = wm * kTM * 16 + i * 16 + (lane & 15);
#pragma unroll
      for (int j = 0; j < kTN; ++j) {
        const int n = wn * kTN * 16 + j * 16 + (lane >> 4) * 4;
        epi.load_elem(m < rows ? m : 0, n < cols ? n : 0, row[i], el[i][j]);
      }
    }
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      const int m = wm * kTM * 16 + i * 16 + (lane & 15);
      if (m >= rows) continue;
#pragma unroll
      for (int j = 0; j < kTN; ++j) {
        const int n = wn * kTN * 16 + j * 16 + (lane >> 4) * 4;
        if (n >= cols) continue;
        float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
        epi.apply(m, n, v, row[i], col[j], el[i][j]);
      }
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
