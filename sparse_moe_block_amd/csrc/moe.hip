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
#include <atomic>

#include "common.h"
#include "gemm_core.h"
#include "kernels.h"

namespace zaya {

// ----------------------------------------------------------------------------- buckets

// One workgroup per kBucketTok tokens, all independent. The router leaves per-class
// token counts of each of its 16-token tiles (counts[c * ld + r], ld a multiple of 4).
// Thread (class c, segment g) sums row c over its segment of the tiles with 16-byte
// loads issued eight at a time (indices clamped, sums masked, so nothing waits inside a
// batch), separately for the tiles before this workgroup's chunk and for all tiles; the
// segments are then added in LDS. That gives every expert's offset (an exclusive scan
// over the experts' totals) and its tokens in earlier chunks. The chunk's tokens are
// placed by their ballot rank within the wave plus the counts of the earlier waves, so
// ids stay ascending within an expert. Skip tokens (class E) get no slot.
constexpr int kBucketTok = 1024;

template <int CB>  // classes the thread grid covers (E <= CB)
__global__ __launch_bounds__(kBucketTok) void bucket_kernel(const int32_t* __restrict__ cls,
                                                            const int32_t* __restrict__ counts, int ld, int ntok,
                                                            int E, int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ ids) {
  constexpr int NW = kBucketTok / 64, SEG = kBucketTok / CB;
  __shared__ int part[2][CB][SEG + 1];  // per (class, segment): counts before the chunk, totals
  __shared__ int base[32];              // expert offset + its tokens in earlier chunks
  __shared__ int wcnt[NW][32];          // the chunk's tokens per expert, per wave
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nrw = (ntok + kRouterTokens - 1) / kRouterTokens;
  const int r_end = blockIdx.x * (kBucketTok / kRouterTokens);  // router tiles before this chunk
  const int t = blockIdx.x * kBucketTok + tid;
  const int k = t < ntok ? cls[t] : -1;
  {
    const int c = tid / SEG, g = tid % SEG;
    const int nq = ld / 4;                  // 16-byte chunks per row
    const int per = (nq + SEG - 1) / SEG;   // chunks per segment
    const int q0 = g * per, q1 = min(q0 + per, nq);
    const int4* row = reinterpret_cast<const int4*>(counts + (size_t)min(c, E - 1) * ld);
    int bef = 0, tot = 0;
    for (int qb = q0; qb < q1; qb += 8) {
      int4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = row[min(qb + j, nq - 1)];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 4 * (qb + j);
        const int x[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool in = qb + j < q1 && r + i < nrw;
          tot += in ? x[i] : 0;
          bef += in && r + i < r_end ? x[i] : 0;
        }
      }
    }
    part[0][c][g] = bef;
    part[1][c][g] = tot;
  }
  // ranks of this wave's tokens among the same expert's
  const unsigned long long lt = (1ull << lane) - 1ull;
  int rank = 0, mine = 0;
  for (int e = 0; e < E; ++e) {
    const unsigned long long m = __ballot(k == e);
    if (lane == e) mine = __popcll(m);
    if (k == e) rank = __popcll(m & lt);
  }
  if (lane < E) wcnt[wave][lane] = mine;
  __syncthreads();
  if (wave == 0) {
    int bef = 0, tot = 0;
    if (lane < E)
      for (int g = 0; g < SEG; ++g) {
        bef += part[0][lane][g];
        tot += part[1][lane][g];
      }
    int incl = tot;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    if (lane < E) base[lane] = incl - tot + bef;
    if (blockIdx.x == 0) {
      if (lane < E) offsets[lane] = incl - tot;
      if (lane == E - 1) offsets[E] = incl;
    }
  }
  __syncthreads();
  if (k >= 0 && k < E) {
    int pos = base[k] + rank;
    for (int w = 0; w < wave; ++w) pos += wcnt[w][k];
    ids[pos] = t;
  }
}

int bucket_counts_ld(int ntok) { return ((ntok + kRouterTokens - 1) / kRouterTokens + 3) / 4 * 4; }

hipError_t launch_bucket(const int32_t* cls, const int32_t* counts, int ntok, int E, int32_t* offsets, int32_t* ids,
                         hipStream_t s) {
  if (ntok <= 0) return hipSuccess;
  if (E > 31) return hipErrorInvalidValue;
  const dim3 grid((ntok + kBucketTok - 1) / kBucketTok);
  const int ld = bucket_counts_ld(ntok);
  if (E <= 16)
    hipLaunchKernelGGL(bucket_kernel<16>, grid, dim3(kBucketTok), 0, s, cls, counts, ld, ntok, E, offsets, ids);
  else
    hipLaunchKernelGGL(bucket_kernel<32>, grid, dim3(kBucketTok), 0, s, cls, counts, ld, ntok, E, offsets, ids);
  return hipGetLastError();
}

// Buckets of at most 64 tokens, in the calling workgroup's LDS (wave 0 forms them,
// then every thread waits): per expert, in expert order, a ballot of the tokens of that
// class gives the count (the running sum is the offset) and each token's rank among the
// earlier tokens of its expert gives its slot, so ids stay ascending within an expert.
// Workgroup 0 also stores them for the kernels that follow. Returns the LDS tables.
struct SmallBuckets {
  int off[33];
  int ids[64];
};
__device__ __forceinline__ void small_buckets(const int32_t* __restrict__ cls, int ntok, int E, SmallBuckets& sb,
                                              int32_t* offsets_out, int32_t* ids_out) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int c = lane < ntok ? cls[lane] : -1;
    const unsigned long long lt = (1ull << lane) - 1ull;
    int run = 0;
    for (int e = 0; e < E; ++e) {
      const unsigned long long m = __ballot(c == e);
      if (lane == 0) sb.off[e] = run;
      if (c == e) sb.ids[run + __popcll(m & lt)] = lane;
      run += __popcll(m);
    }
    if (lane == 0) sb.off[E] = run;
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    if ((int)threadIdx.x <= E) offsets_out[threadIdx.x] = sb.off[threadIdx.x];
    if ((int)threadIdx.x < sb.off[E]) ids_out[threadIdx.x] = sb.ids[threadIdx.x];
  }
}

// ----------------------------------------------------------------------------- packed expert weights
//
// A grouped-GEMM item streams the K slices (128 bytes of a row) of 128 weight rows. In
// the row-major layout those 128 x 128 bytes lie 128 row lengths apart, so each slice
// load opens as many DRAM pages; packed, the slices of a 128-row group follow one
// another (group-major, then slice, then row), so an item reads one contiguous run of
// HBM. Group j of W_gu holds the rows a gate/up item uses, in its order: 16-row blocks
// alternating gate (rows 64 j + 16 b ..) and up (rows I + 64 j + 16 b ..). Group g of
// W_dn holds rows 128 g .. 128 g + 127. Both are plain permutations of 16-byte chunks.
template <bool GATEUP>
__global__ __launch_bounds__(256) void pack_experts_kernel(const char* __restrict__ src, char* __restrict__ dst,
                                                           size_t nchunks, int rows_e, int row_bytes, int I) {
  const int ns = row_bytes / kPackSliceBytes;  // slices per row
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nchunks; i += (size_t)gridDim.x * blockDim.x) {
    const int c = (int)(i & 7);
    const int q = (int)((i >> 3) % kPackRows);
    const size_t gs = i / (8 * kPackRows);  // (expert, group, slice)
    const int s = (int)(gs % ns);
    const size_t eg = gs / ns;
    const int ng = rows_e / kPackRows;
    const int grp = (int)(eg % ng), e = (int)(eg / ng);
    int row;
    if constexpr (GATEUP) {
      const int blk = q >> 4;
      row = ((blk & 1) ? I : 0) + 64 * grp + (blk >> 1) * 16 + (q & 15);
    } else {
      row = grp * kPackRows + q;
    }
    const size_t from = ((size_t)e * rows_e + row) * row_bytes + (size_t)s * kPackSliceBytes + c * 16;
    *reinterpret_cast<u32x4*>(dst + i * 16) = *reinterpret_cast<const u32x4*>(src + from);
  }
}

template <typename T>
hipError_t launch_pack_experts(const T* Wgu, const T* Wdn, T* Pgu, T* Pdn, int E, int H, int I, hipStream_t s) {
  if (E <= 0) return hipSuccess;
  if ((2 * I) % kPackRows || H % kPackRows || (H * (int)sizeof(T)) % kPackSliceBytes ||
      (I * (int)sizeof(T)) % kPackSliceBytes)
    return hipErrorInvalidValue;
  const size_t ngu = (size_t)E * 2 * I * H * sizeof(T) / 16, ndn = (size_t)E * H * I * sizeof(T) / 16;
  const int grid = 256 * 8;
  hipLaunchKernelGGL(pack_experts_kernel<true>, dim3(grid), dim3(256), 0, s, reinterpret_cast<const char*>(Wgu),
                     reinterpret_cast<char*>(Pgu), ngu, 2 * I, H * (int)sizeof(T), I);
  hipLaunchKernelGGL(pack_experts_kernel<false>, dim3(grid), dim3(256), 0, s, reinterpret_cast<const char*>(Wdn),
                     reinterpret_cast<char*>(Pdn), ndn, H, I * (int)sizeof(T), I);
  return hipGetLastError();
}

// FP8 codes: destination 16-byte chunk i holds chunk i % 4 of the 64-byte step s of row
// r (i / 4 % 16) of block b, expert e: source row 16 b + r, bytes 64 s + 16 (i % 4).
__global__ __launch_bounds__(256) void pack_experts_f8_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                              size_t nchunks, int rows_e, int row_bytes) {
  const int ns = row_bytes / kF8PackStep;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nchunks; i += (size_t)gridDim.x * blockDim.x) {
    const int c = (int)(i & 3);
    const int r = (int)((i >> 2) % kF8PackRows);
    const size_t bs = i / (4 * kF8PackRows);  // (expert, block, step)
    const int st = (int)(bs % ns);
    const size_t eb = bs / ns;
    const int nb = rows_e / kF8PackRows;
    const int blk = (int)(eb % nb), e = (int)(eb / nb);
    const size_t from = ((size_t)e * rows_e + (size_t)blk * kF8PackRows + r) * row_bytes + (size_t)st * kF8PackStep + c * 16;
    *reinterpret_cast<u32x4*>(dst + i * 16) = *reinterpret_cast<const u32x4*>(src + from);
  }
}

hipError_t launch_pack_experts_f8(const uint8_t* Wgu, const uint8_t* Wdn, uint8_t* Pgu, uint8_t* Pdn, int E, int H,
                                  int I, hipStream_t s) {
  if (E <= 0) return hipSuccess;
  if ((2 * I) % kF8PackRows || H % kF8PackRows || H % kF8PackStep || I % kF8PackStep) return hipErrorInvalidValue;
  const size_t ngu = (size_t)E * 2 * I * H / 16, ndn = (size_t)E * H * I / 16;
  hipLaunchKernelGGL(pack_experts_f8_kernel, dim3(2048), dim3(256), 0, s, Wgu, Pgu, ngu, 2 * I, H);
  hipLaunchKernelGGL(pack_experts_f8_kernel, dim3(2048), dim3(256), 0, s, Wdn, Pdn, ndn, H, I);
  return hipGetLastError();
}

template hipError_t launch_pack_experts<bf16_t>(const bf16_t*, const bf16_t*, bf16_t*, bf16_t*, int, int, int,
                                                 hipStream_t);
template hipError_t launch_pack_experts<float>(const float*, const float*, float*, float*, int, int, int,
                                                hipStream_t);

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
//
// Tail split. The items run in rounds of `slots` (the workgroups resident on the whole
// chip at once); a last round of a few items would leave most of the chip idle for an
// item's whole duration (560 down items on 512 slots: a second round of 48). When
// split > 1 and the items past the last full round, split into `split` column parts
// each, fit one round, those parts are items of their own: every XCD runs its share of
// full items (in contiguous runs, as above), then its share of the parts. part_out is
// the column part (0 .. split - 1) of such an item, or -1 for a whole item.
__device__ __forceinline__ bool moe_item(const int32_t* __restrict__ off, int E, int BM, int ntn, int slots, int split,
                                         int& e_out, int& r0_out, int& n_out, int& nt_out, int& part_out) {
  // Every wave finds the item on its own: lane e < E reads offsets e and e + 1 (one
  // memory round trip; the offsets may live in LDS or in global memory), the row-tile
  // counts are scanned across lanes, and the expert holding the item is the first lane
  // whose running tile count passes it. E < 64 (checked by the host).
  const int lane = threadIdx.x & 63;
  const int o0 = off[min(lane, E)], o1 = off[min(lane + 1, E)];
  const int n = lane < E ? o1 - o0 : 0;
  const int mt = (n + BM - 1) / BM;
  int incl = mt;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
  const int tiles = __shfl(incl, 63, 64);
  const int n_real = tiles * ntn;
  const int x = (int)blockIdx.x % 8, k = (int)blockIdx.x / 8;
  const int nfull = slots > 0 ? n_real / slots * slots : n_real;  // slots: a multiple of 8
  const int nsub = (n_real - nfull) * split;
  int item;
  part_out = -1;
  if (split > 1 && nsub > 0 && nsub <= slots) {
    const int fx = nfull / 8, spx = (nsub + 7) / 8;
    if (k < fx) {
      item = x * fx + k;
    } else {
      const int sub = x * spx + (k - fx);
      if (k - fx >= spx || sub >= nsub) return false;
      item = nfull + sub / split;
      part_out = sub % split;
    }
  } else {
    const int per = (n_real + 7) / 8;
    if (k >= per) return false;
    item = x * per + k;
    if (item >= n_real) return false;
  }
  const unsigned long long past = __ballot(lane < E && incl * ntn > item);
  const int e = __ffsll((long long)past) - 1;
  const int mt_e = __shfl(mt, e, 64);
  item -= (__shfl(incl, e, 64) - mt_e) * ntn;
  e_out = e;
  nt_out = item / mt_e;
  r0_out = (item % mt_e) * BM;
  n_out = __shfl(n, e, 64);
  return true;
}

// Grid for a grouped GEMM: an upper bound on the items, rounded to the 8 XCDs, plus
// the split tail's parts (at most one round of `slots`).
static inline int moe_grid(int ntok, int E, int BM, int ntn, int slots = 0) {
  const int nmax = ((ntok + BM - 1) / BM + E) * ntn;
  return 8 * ((nmax + 7) / 8) + 8 * ((slots + 7) / 8);
}

// One gate/up item: Tile::kBN weight rows = kBN / 2 activation columns starting at c0,
// gate and up in alternating 16-row blocks; the item starts at row q0 of 128-row group
// grp and may run on into the following groups (each group's rows are in that order,
// packed or not, and consecutive groups hold consecutive activation columns).
template <typename T, class Tile>
__device__ __forceinline__ void gateup_item(const MoeArgs<T>& a, const int32_t* __restrict__ ids, char* smem, int e,
                                            int base, int rows, int grp, int q0) {
  static_assert(Tile::kTN % 2 == 0, "each wave needs gate/up pairs");
  static_assert(Tile::kRowBytes == kPackSliceBytes, "packed slices are the tile's K slices");
  const int c0 = grp * (kPackRows / 2) + q0 / 2;  // activation columns [c0, c0 + kBN / 2)
  Tile t;
  const T* Wg = a.W_gu + (size_t)e * 2 * a.I * a.H;
  if (a.packed) {  // item row r is row (q0 + r) % 128 of packed group grp + (q0 + r) / 128
    t.set_b([&](int r) -> const T* {
      return Wg + (size_t)(grp + (q0 + r) / kPackRows) * kPackRows * a.H + (size_t)((q0 + r) % kPackRows) * Tile::kBK;
    });
    t.bstride = (size_t)kPackRows * Tile::kRowBytes;
  } else {
    t.set_b([&](int r) -> const T* {
      const int blk = r >> 4, w16 = r & 15;
      const int row = ((blk & 1) ? a.I : 0) + c0 + (blk >> 1) * 16 + w16;
      return Wg + (size_t)row * a.H;
    });
  }
  t.set_a([&](int r) -> const T* { return a.hn + (size_t)ids[base + min(r, rows - 1)] * a.H; });
  t.run(smem, a.H / Tile::kBK);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / Tile::kWN, wn = wave % Tile::kWN;
#pragma unroll
  for (int i = 0; i < Tile::kTM; ++i) {
    const int m = wm * Tile::kTM * 16 + i * 16 + (lane & 15);
    if (m >= rows) continue;
    T* nrow = a.neurons + (size_t)(base + m) * a.I;
#pragma unroll
    for (int pp = 0; pp < Tile::kTN / 2; ++pp) {
      const int col = c0 + (wn * (Tile::kTN / 2) + pp) * 16 + (lane >> 4) * 4;
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

// BN weight rows per item (BN / 128 whole 128-row groups: BN / 2 activation columns);
// with SPLIT > 1 the tail items of moe_item run as SPLIT parts of BN / SPLIT rows (waves
// stacked along the rows when a part is too narrow to give every wave gate/up pairs).
template <typename T, int BM, int WM, int WN, int BN = 128, int SPLIT = 1>
__global__ __launch_bounds__(WM* WN * 64)
__attribute__((amdgpu_waves_per_eu(GemmTile<T, BM, BN, WM, WN>::kWavesPerEU))) void moe_gateup_kernel(MoeArgs<T> a) {
  static_assert(BN % kPackRows == 0, "a gate/up item is whole 128-row groups");
  using Tile = GemmTile<T, BM, BN, WM, WN, (BM <= 16 && kStreamFewRows)>;  // 16-row items: one item per weight tile
  constexpr bool kNarrow = BN / SPLIT < WN * 32;
  using Part = GemmTile<T, BM, BN / SPLIT, kNarrow ? WM * WN : WM, kNarrow ? 1 : WN, (BM <= 16 && kStreamFewRows)>;
  __shared__ __attribute__((aligned(16))) char smem[Tile::kLdsBytes];
  __shared__ SmallBuckets sb;
  const int32_t* off = a.offsets;
  const int32_t* ids = a.ids;
  if (a.cls) {  // few tokens: the buckets are formed here
    small_buckets(a.cls, a.ntok, a.E, sb, a.offsets_out, a.ids_out);
    off = sb.off;
    ids = sb.ids;
  }
  int e, r0, n_e, j, part;  // j: item along the rows (groups j * BN / 128 ..)
  if (!moe_item(off, a.E, BM, a.I / (BN / 2), SPLIT > 1 ? a.slots : 0, SPLIT, e, r0, n_e, j, part)) return;
  const int base = off[e] + r0;
  const int rows = min(BM, n_e - r0);
  if (SPLIT > 1 && part >= 0)
    gateup_item<T, Part>(a, ids, smem, e, base, rows, j * (BN / kPackRows), part * (BN / SPLIT));
  else
    gateup_item<T, Tile>(a, ids, smem, e, base, rows, j * (BN / kPackRows), 0);
}

// Down-projection epilogue: y = rnd(sum), routed = rnd(w * y), mlp = rnd(rnd(routed + hsb)
// * hss), out = f32(f32(h + rb) * rs) + mlp, for the item's token rows (bucket order) and
// output columns n0 + n. The row's token and weight are read first, then the stream rows
// and the merge vectors, all before the first result.
template <typename T>
struct EpiDownMerge {
  const MoeArgs<T>& a;
  int base, n0;
  struct Row {
    int tok;
    float w;
  };
  struct Col {
    float b1[4], s1[4], b2[4], s2[4];
  };
  struct Elem {
    float hv[4];
  };
  __device__ __forceinline__ void load_row(int m, Row& r) const {
    r.tok = a.ids[base + m];
    r.w = Act<T>::tof(a.wts[r.tok]);
  }
  __device__ __forceinline__ void load_col(int nl, Col& c) const {
    const int n = n0 + nl;
    load4(a.hsb + n, c.b1);
    load4(a.hss + n, c.s1);
    load4(a.rb + n, c.b2);
    load4(a.rs + n, c.s2);
  }
  __device__ __forceinline__ void load_elem(int, int nl, const Row& r, Elem& e) const {
    load4(a.h + (size_t)r.tok * a.H + n0 + nl, e.hv);
  }
  __device__ __forceinline__ void apply(int, int nl, const float* v, const Row& r, const Col& c, const Elem& e) const {
    const int n = n0 + nl;
    float ro[4], mo[4], o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float y = Act<T>::rnd(v[q]);
      ro[q] = Act<T>::rnd(r.w * y);
      mo[q] = Act<T>::rnd(Act<T>::rnd(ro[q] + c.b1[q]) * c.s1[q]);
      o[q] = fadd(fmul(fadd(e.hv[q], c.b2[q]), c.s2[q]), mo[q]);
    }
    store4(a.out + (size_t)r.tok * a.H + n, o);
    if (a.routed_tap) store4(a.routed_tap + (size_t)r.tok * a.H + n, ro);
    if (a.mlp_tap) store4(a.mlp_tap + (size_t)r.tok * a.H + n, mo);
  }
};

// One down item: output columns n0 .. n0 + Tile::kBN of the item's token rows.
template <typename T, class Tile>
__device__ __forceinline__ void down_item(const MoeArgs<T>& a, char* smem, int e, int base, int rows, int n0) {
  Tile t;
  t.set_a([&](int r) -> const T* { return a.neurons + (size_t)(base + min(r, rows - 1)) * a.I; });
  const T* Wd = a.W_dn + (size_t)e * a.H * a.I;
  if (a.packed) {  // output row n is row n % 128 of packed group n / 128
    t.set_b([&](int r) -> const T* {
      return Wd + (size_t)((n0 + r) / kPackRows) * kPackRows * a.I + (size_t)((n0 + r) % kPackRows) * Tile::kBK;
    });
    t.bstride = (size_t)kPackRows * Tile::kRowBytes;
  } else {
    t.set_b([&](int r) -> const T* { return Wd + (size_t)(n0 + r) * a.I; });
  }
  t.run(smem, a.I / Tile::kBK);
  t.epilogue_loaded(EpiDownMerge<T>{a, base, n0}, rows);
}

// BN output columns per item; with SPLIT > 1 the tail items of moe_item run as SPLIT
// parts of BN / SPLIT columns.
template <typename T, int BM, int WM, int WN, int BN = 128, int SPLIT = 1>
__global__ __launch_bounds__(WM* WN * 64)
__attribute__((amdgpu_waves_per_eu(GemmTile<T, BM, BN, WM, WN>::kWavesPerEU))) void moe_down_kernel(MoeArgs<T> a) {
  using Tile = GemmTile<T, BM, BN, WM, WN, (BM <= 16 && kStreamFewRows)>;  // 16-row items: one item per weight tile
  constexpr bool kNarrow = BN / SPLIT < WN * 16;  // then the part's waves stack along the rows
  using Part = GemmTile<T, BM, BN / SPLIT, kNarrow ? WM * WN : WM, kNarrow ? 1 : WN, (BM <= 16 && kStreamFewRows)>;
  __shared__ __attribute__((aligned(16))) char smem[Tile::kLdsBytes];
  int e, r0, n_e, c, part;
  if (!moe_item(a.offsets, a.E, BM, a.H / BN, SPLIT > 1 ? a.slots : 0, SPLIT, e, r0, n_e, c, part)) return;
  const int base = a.offsets[e] + r0;
  const int rows = min(BM, n_e - r0);
  if (SPLIT > 1 && part >= 0)
    down_item<T, Part>(a, smem, e, base, rows, c * BN + part * (BN / SPLIT));
  else
    down_item<T, Tile>(a, smem, e, base, rows, c * BN);
}

// Workgroups of the 128-row expert tiles resident on the current device at once (two
// 4-wave or one 8-wave workgroup per CU), a multiple of 8; 0 if the device cannot be
// queried.
static int moe_slots(int waves) {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];  // per device: 0 = not yet asked, else CUs + 1
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  const int c = dev >= 0 && dev < kMaxDev ? cache[dev].load(std::memory_order_relaxed) : 0;
  if (c > 0) {
    cus = c - 1;
  } else {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (dev >= 0 && dev < kMaxDev) cache[dev].store(cus + 1, std::memory_order_relaxed);
  }
  return (cus * (8 / waves)) / 8 * 8;  // eight waves of a CU are resident at once
}

template <typename T, int BM, int WM, int WN, int BN = 128, int SPLIT = 1>
static hipError_t launch_gateup_cfg(const MoeArgs<T>& a0, hipStream_t s) {
  MoeArgs<T> a = a0;
  a.slots = SPLIT > 1 ? moe_slots(WM * WN) : 0;
  hipLaunchKernelGGL((moe_gateup_kernel<T, BM, WM, WN, BN, SPLIT>), dim3(moe_grid(a.ntok, a.E, BM, a.I / (BN / 2), a.slots)),
                     dim3(WM * WN * 64), 0, s, a);
  return hipGetLastError();
}

template <typename T, int BM, int WM, int WN, int BN = 128, int SPLIT = 1>
static hipError_t launch_down_cfg(const MoeArgs<T>& a0, hipStream_t s) {
  MoeArgs<T> a = a0;
  a.slots = SPLIT > 1 ? moe_slots(WM * WN) : 0;
  hipLaunchKernelGGL((moe_down_kernel<T, BM, WM, WN, BN, SPLIT>), dim3(moe_grid(a.ntok, a.E, BM, a.H / BN, a.slots)),
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
  return launch_gateup_cfg<T, 128, 2, 2, 128, 2>(a, s);
}

template <typename T>
hipError_t launch_moe_down(const MoeArgs<T>& a, hipStream_t s) {
  if (a.ntok <= 0) return hipSuccess;
  if (a.ntok <= 32 * a.E) return launch_down_cfg<T, 16, 1, 4, 64>(a, s);
  return launch_down_cfg<T, 128, 2, 2, 128, 4>(a, s);
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
  __shared__ SmallBuckets sb;
  const int32_t* off = a.offsets;
  const int32_t* ids = a.ids;
  if (GATEUP && a.cls) {  // few tokens: the buckets are formed here
    small_buckets(a.cls, a.ntok, a.E, sb, a.offsets_out, a.ids_out);
    off = sb.off;
    ids = sb.ids;
  }
  int e, r0, n_e, j;
  int part;
  if (!moe_item(off, a.E, kF8Tok, ntn, 0, 1, e, r0, n_e, j, part)) return;
  const int base = off[e] + r0;
  const int rows = min(kF8Tok, n_e - r0);
  const int pitch = K * 2 + 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, grp = lane >> 4;

  // weight rows of this lane (byte pointers at its 16-byte column) and the first loads
  const uint8_t* W = reinterpret_cast<const uint8_t*>(GATEUP ? (const void*)a.W_gu : (const void*)a.W_dn) +
                     (size_t)e * (GATEUP ? 2 * (size_t)a.I * a.H : (size_t)a.H * a.I);
  const int n_row = 64 * j + 16 * wave + r16;  // gate row (gate/up) or output row (down)
  const int up_row = GATEUP ? a.I + n_row : n_row;
  // packed codes: the 16-row block's step s is one KiB, this lane's row at 64 r16
  const size_t wstep = a.packed ? (size_t)kF8PackRows * kF8PackStep : (size_t)kF8PackStep;
  auto wrow = [&](int row) -> const uint8_t* {
    return a.packed ? W + (size_t)(row - r16) * K + r16 * kF8PackStep + grp * 16 : W + (size_t)row * K + grp * 16;
  };
  const uint8_t* w0 = wrow(n_row);
  const uint8_t* w1 = wrow(up_row);
  const int nds = K / 64;
  auto wload = [](const uint8_t* p) -> u32x4 {
    if constexpr (STREAM) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    else return *reinterpret_cast<const u32x4*>(p);
  };
  u32x4 q0[kF8Ahead], q1[kF8Ahead];
  auto prefetch_w = [&]() {
#pragma unroll
    for (int p = 0; p < kF8Ahead; ++p) {
      const int s = min(p, nds - 1);
      q0[p] = wload(w0 + (size_t)s * wstep);
      if (GATEUP) q1[p] = wload(w1 + (size_t)s * wstep);
    }
  };

  // Stage the tile's token rows, 16 chunks of 16 bytes per thread a batch; the weights'
  // first loads go out right behind the last batch's, so that batch waits for its own
  // loads only and the weight loads are the only ones in flight when the products start.
  // Only the tile's rows are loaded: the products of the rows past them read whatever LDS
  // holds, and only those tokens' outputs (never stored) depend on them.
  {
    constexpr int kSB = 16;
    const int cpr = K / 8;  // 16-byte chunks per row
    const int nch = rows * cpr;
    const int nb = (nch + kSB * 256 - 1) / (kSB * 256);  // batches, the same for every thread
    u32x4 v[kSB];
    auto load_batch = [&](int c0) {
#pragma unroll
      for (int u = 0; u < kSB; ++u) {
        const int ch = min(c0 + u * 256, nch - 1);
        const int r = ch / cpr, cc = ch % cpr;
        const bf16_t* src = GATEUP ? a.hn + (size_t)ids[base + r] * a.H : a.neurons + (size_t)(base + r) * a.I;
        v[u] = *reinterpret_cast<const u32x4*>(src + cc * 8);
      }
    };
    auto store_batch = [&](int c0) {
#pragma unroll
      for (int u = 0; u < kSB; ++u) {
        const int ch = c0 + u * 256;
        if (ch < nch) *reinterpret_cast<u32x4*>(xs + (ch / cpr) * pitch + (ch % cpr) * 16) = v[u];
      }
    };
    for (int bi = 0; bi + 1 < nb; ++bi) {
      load_batch((int)threadIdx.x + bi * kSB * 256);
      store_batch((int)threadIdx.x + bi * kSB * 256);
    }
    load_batch((int)threadIdx.x + (nb - 1) * kSB * 256);
    prefetch_w();
    store_batch((int)threadIdx.x + (nb - 1) * kSB * 256);
  }
  __syncthreads();

  const char* xrow = xs + r16 * pitch + grp * 32;
  f32x4 acc0 = f32x4{0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
  // step s with the codes in slot p, which is then refilled kF8Ahead steps ahead (past
  // the end: the last step again)
  auto kstep = [&](int s, int p) {
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
    const int sn = min(s + kF8Ahead, nds - 1);
    q0[p] = wload(w0 + (size_t)sn * wstep);
    if (GATEUP) q1[p] = wload(w1 + (size_t)sn * wstep);
    // steps stay in order: the scheduler would otherwise convert later slots' codes
    // first, and wait for every load in flight to do so
    __builtin_amdgcn_sched_barrier(0);
  };
  // Whole rounds of kF8Ahead steps first, with no branch inside: the compiler's wait
  // tracking then sees the same loads in flight on every path and waits for the oldest
  // slot only (with a branch per step it waited for every load in flight, so nothing
  // stayed ahead). Then the remaining steps.
  int s0 = 0;
  for (; s0 + kF8Ahead <= nds; s0 += kF8Ahead) {
#pragma unroll
    for (int p = 0; p < kF8Ahead; ++p) kstep(s0 + p, p);
  }
#pragma unroll
  for (int p = 0; p < kF8Ahead; ++p)
    if (s0 + p < nds) kstep(s0 + p, p);

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
  // dynamic LDS up to what the static bucket tables leave of the CU's 160 KiB
  constexpr int kDyn = 160 * 1024 - 1024;
  static_assert(sizeof(SmallBuckets) <= 1024, "static LDS of the FP8 expert kernel");
  static const hipError_t attr = hipFuncSetAttribute((const void*)moe_f8_kernel<GATEUP, false>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, kDyn);
  static const hipError_t attr_s = hipFuncSetAttribute((const void*)moe_f8_kernel<GATEUP, true>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kDyn);
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
