// Grouped-query attention over the CCA queries/keys/values.
//
// Semantics ("The API / support()": attention_scores masked, softmax, pattern times
// values; "Config": 8 query heads over 2 KV heads; "Queries and keys are convolved
// ..." for the window): query head h reads KV head h / (nh/nkv); score = q.k / sqrt(d);
// key k is visible from query q iff p_k <= p_q and, with a window W >= 0,
// p_q - p_k <= W. Softmax in fp32 (online, base 2), output rounded to act.
//
// Prefill kernel: one workgroup per (32-query tile, KV group, sequence) with one wave
// per query head of the group, so the four heads share every K/V tile staged in LDS.
// Both products run on MFMA: S^T = K Q^T (each lane then holds 16 scores of one
// query row, so row statistics need only two cross-lane steps) and O^T = V^T P^T,
// where P is fed straight from the score registers and V is transposed as it is
// written into LDS. Tiles entirely outside the causal/window band are skipped; only
// tiles that cut the band are masked element by element.
//
// Decode kernel (one new token per sequence): split over the cached keys — one
// workgroup per (256-key chunk, KV group, sequence), one wave per query head, K/V
// tiles staged through LDS with 16-byte coalesced loads, scores with one lane per key,
// the weighted sum with one lane per pair of dims — then a combine pass merges the
// chunks' (max, sum, partial output) triples.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace zaya {

constexpr float kLog2e = 1.4426950408889634f;
// Longest run of 64-key tiles one prefill unit handles: 16 for the 32-query kernel, 22
// for the 64-query one (at 4096 tokens: three chunks for the longest query tile, 68.7 us
// for kernel and merge against 72.0 us with four and 81.0 with five).
constexpr int kPrefillChunkTiles = 16;
constexpr int kPrefill64ChunkTiles = 22;

// ----------------------------------------------------------------------------- prefill

// LDS tiles of one 64-key block, unpadded and XOR-swizzled so that the MFMA fragment
// reads (16 rows, one column block) and the tile writes (the transposing V write
// included) each touch distinct banks:
//   K   [64 keys][D]: 16-byte chunk c of key row k stored at chunk c ^ (k % chunks/row);
//   V^T [D][64 keys]: 4-key unit u of dim row d stored at unit u ^ vswz(d) (below).
template <typename T, int D>
struct AttnLds {
  static constexpr int kKeys = 64;
  static constexpr int kKRow = D * (int)sizeof(T);          // bytes per K row
  static constexpr int kKChunksRow = kKRow / 16;
  static constexpr int kVRow = kKeys * (int)sizeof(T);      // bytes per V^T row
  static constexpr int kVUnit = 4 * (int)sizeof(T);         // bytes of a 4-key unit
  static constexpr int kKBytes = kKeys * kKRow;
  static constexpr int kVBytes = D * kVRow;
  static constexpr int kBytes = kKBytes + kVBytes;
  __device__ __forceinline__ static int koff(int key, int chunk) {
    // 16 chunks per row (bf16, d = 128): the key's low bits, plus (key / 16) % 4 in the
    // upper bits, measured faster for the fragment reads (127 vs 115 TB/s)
    const int m = kKChunksRow == 16 ? (key & 15) ^ (((key >> 4) & 3) << 2) : (key & (kKChunksRow - 1));
    return key * kKRow + ((chunk ^ m) << 4);
  }
  // Measured on gfx950 (fragment reads: 16 dim rows x 4 unit columns per lane group;
  // transposing writes: 8 rows of one unit per lane): this mask reads at ~97 TB/s over
  // the chip where ((d / 8) % 16) ^ (d % 8 * 2) managed ~65, and writes as fast.
  __device__ __forceinline__ static int vswz(int d) { return (((d >> 1) & 7) << 1) ^ ((d >> 4) & 7); }
  __device__ __forceinline__ static int voff(int d, int unit) { return d * kVRow + (unit ^ vswz(d)) * kVUnit; }
};

// Global -> registers for one 64-key tile: K rows as 16-byte chunks, V as 4-key x 8-dim
// blocks (so the transposed LDS write packs four keys per store).
template <typename T, int D>
struct TileRegs {
  static constexpr int kElem16 = 16 / (int)sizeof(T);            // elements per 16 bytes
  static constexpr int kKChunks = 64 * D / kElem16;              // 16-byte chunks in the K tile
  static constexpr int kVTasks = 16 * (D / 8);                   // (key quad, 8-dim block) tasks
};

template <typename T, int D, int NT>
__device__ __forceinline__ void attn_load_tile(const T* Kb, const T* Vb, int k0, int kvalid, uint4* kr, uint4* vr) {
  using TR = TileRegs<T, D>;
  constexpr int KC = (TR::kKChunks + NT - 1) / NT;
  constexpr int VT = (TR::kVTasks + NT - 1) / NT;
  constexpr int per_row = D / TR::kElem16;
#pragma unroll
  for (int i = 0; i < KC; ++i) {
    const int c = threadIdx.x + i * NT;
    const int key = c / per_row, col = (c % per_row) * TR::kElem16;
    kr[i] = (c < TR::kKChunks && k0 + key < kvalid)
                ? *reinterpret_cast<const uint4*>(Kb + (size_t)(k0 + key) * D + col)
                : make_uint4(0, 0, 0, 0);
  }
  // V: task = (quad q4, block db8): keys 4*q4..+3, dims 8*db8..+7 -> 4 rows x (8 elements)
  constexpr int VW = 8 * (int)sizeof(T) / 16;  // 16-byte words per 8 elements (1 or 2)
#pragma unroll
  for (int i = 0; i < VT; ++i) {
    const int task = threadIdx.x + i * NT;
    const int q4 = task / (D / 8), db8 = task % (D / 8);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int w = 0; w < VW; ++w) {
        const int key = 4 * q4 + kk;
        vr[(i * 4 + kk) * VW + w] = (task < TR::kVTasks && k0 + key < kvalid)
                                        ? *reinterpret_cast<const uint4*>(Vb + (size_t)(k0 + key) * D + db8 * 8 + w * TR::kElem16)
                                        : make_uint4(0, 0, 0, 0);
      }
  }
}

template <typename T, int D, int NT>
__device__ __forceinline__ void attn_store_tile(char* lds, const uint4* kr, const uint4* vr) {
  using TR = TileRegs<T, D>;
  using L = AttnLds<T, D>;
  constexpr int KC = (TR::kKChunks + NT - 1) / NT;
  constexpr int VT = (TR::kVTasks + NT - 1) / NT;
  constexpr int per_row = D / TR::kElem16;
  constexpr int VW = 8 * (int)sizeof(T) / 16;
#pragma unroll
  for (int i = 0; i < KC; ++i) {
    const int c = threadIdx.x + i * NT;
    if (c < TR::kKChunks) {
      const int key = c / per_row, chunk = c % per_row;
      *reinterpret_cast<uint4*>(lds + L::koff(key, chunk)) = kr[i];
    }
  }
  char* vt = lds + L::kKBytes;
#pragma unroll
  for (int i = 0; i < VT; ++i) {
    const int task = threadIdx.x + i * NT;
    if (task >= TR::kVTasks) continue;
    const int q4 = task / (D / 8), db8 = task % (D / 8);
    // element j (0..7) of key kk lives in word (kk, j / kElem16), slot j % kElem16
    const T* e[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) e[kk] = reinterpret_cast<const T*>(&vr[(i * 4 + kk) * VW]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      T* dst = reinterpret_cast<T*>(vt + L::voff(db8 * 8 + j, q4));
      if constexpr (sizeof(T) == 2) {
        uint2 w;
        w.x = (uint32_t)e[0][j] | ((uint32_t)e[1][j] << 16);
        w.y = (uint32_t)e[2][j] | ((uint32_t)e[3][j] << 16);  // keys 4 q4 .. 4 q4 + 3
        *reinterpret_cast<uint2*>(dst) = w;
      } else {
        *reinterpret_cast<float4*>(dst) = make_float4(e[0][j], e[1][j], e[2][j], e[3][j]);
      }
    }
  }
}

// V^T fragment for dim row drow and the 32-key block c: keys 32c + 4 grp .. +3 then
// 32c + 16 + 4 grp .. +3 (the order the score registers hold them in).
template <typename T, int D>
__device__ __forceinline__ typename Mfma<T>::frag load_vt_frag(const char* vt, int drow, int c, int grp) {
  using L = AttnLds<T, D>;
  typename Mfma<T>::frag f;
  if constexpr (sizeof(T) == 2) {
    const uint2 lo = *reinterpret_cast<const uint2*>(vt + L::voff(drow, 8 * c + grp));
    const uint2 hi = *reinterpret_cast<const uint2*>(vt + L::voff(drow, 8 * c + 4 + grp));
    f.v = make_uint4(lo.x, lo.y, hi.x, hi.y);
  } else {
    f.a = *reinterpret_cast<const float4*>(vt + L::voff(drow, 8 * c + grp));
    f.b = *reinterpret_cast<const float4*>(vt + L::voff(drow, 8 * c + 4 + grp));
  }
  return f;
}

// K fragment of key row `key`, d elements [32 dc + 8 grp, +8).
template <typename T, int D>
__device__ __forceinline__ typename Mfma<T>::frag attn_k_frag(const char* kbuf, int key, int dc, int grp) {
  using L = AttnLds<T, D>;
  constexpr int CPF = 8 * (int)sizeof(T) / 16;  // 16-byte chunks per fragment (1 or 2)
  const int c0 = (dc * 32 + grp * 8) * (int)sizeof(T) / 16;
  typename Mfma<T>::frag f;
  if constexpr (CPF == 1) {
    f.v = *reinterpret_cast<const uint4*>(kbuf + L::koff(key, c0));
  } else {
    f.a = *reinterpret_cast<const float4*>(kbuf + L::koff(key, c0));
    f.b = *reinterpret_cast<const float4*>(kbuf + L::koff(key, c0 + 1));
  }
  return f;
}

// Key-tile range of query tile qblk of sequence b, and how it is split into chunks:
// chunk c of nc covers tiles [kt_begin + c*n/nc, kt_begin + (c+1)*n/nc).
struct QTile {
  int q0, nq, qp_min, qp_max, kt_begin, n, nc;
};

template <int QW = 32>
__device__ __forceinline__ QTile qtile(int qblk, int S, int L0, int W, int NC) {
  QTile r;
  r.q0 = qblk * QW;
  r.nq = min(QW, S - r.q0);
  r.qp_min = L0 + r.q0;
  r.qp_max = L0 + r.q0 + r.nq - 1;
  const int klo = W >= 0 ? max(0, r.qp_min - W) : 0;
  r.kt_begin = klo / 64;
  r.n = r.qp_max / 64 + 1 - r.kt_begin;
  r.nc = min(NC, r.n);  // short ranges split too: their small units fill the last round
  return r;
}

// One unit = (query tile of 32 tokens, chunk of its key tiles, KV group, sequence).
// Units are numbered so the latest (heaviest) query tiles come first. A query tile
// whose keys fit one chunk writes its output directly; otherwise each chunk writes
// (unnormalised output, running max, running sum) per row for the combine pass.
template <typename T, int D, int G>
__global__ __launch_bounds__(64 * G) __attribute__((amdgpu_waves_per_eu(2))) void attn_prefill_kernel(
    AttnArgs<T> a, float* __restrict__ part, int NC) {
  using MF = Mfma<T>;
  using frag = typename MF::frag;
  using L = AttnLds<T, D>;
  constexpr int NT = 64 * G;
  constexpr int DC = D / 32;  // 32-wide K chunks of the QK product
  constexpr int DB = D / 16;  // 16-row output blocks of O^T
  __shared__ __attribute__((aligned(16))) char lds[2 * L::kBytes];

  const int nqb = (a.S + 31) / 32;
  const int c = blockIdx.x % NC;
  const int qblk = nqb - 1 - (int)(blockIdx.x / NC);
  const int g = blockIdx.y, b = blockIdx.z;
  const int S = a.S, L0 = cached_len(a.cache_len, b);
  const int W = a.window;
  const QTile qt = qtile(qblk, S, L0, W, NC);
  if (c >= qt.nc) return;
  const int kt0 = qt.kt_begin + c * qt.n / qt.nc;
  const int kt1 = qt.kt_begin + (c + 1) * qt.n / qt.nc;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = g * G + wave;
  const int r16 = lane & 15, grp = lane >> 4;
  const int q0 = qt.q0, qp_min = qt.qp_min, qp_max = qt.qp_max;

  // queries of this head: rows q0 + qb*16 + r16
  frag qf[2][DC];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int t = q0 + qb * 16 + r16;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
      qf[qb][dc] = t < S ? MF::load(a.Q + (((size_t)b * S + t) * a.nh + h) * D + dc * 32 + grp * 8) : MF::zero();
  }

  f32x4 o[2][DB];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db) o[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};

  const int kvalid = L0 + S;
  const T* Kb = a.K + ((size_t)b * a.nkv + g) * a.cap * D;
  const T* Vb = a.V + ((size_t)b * a.nkv + g) * a.cap * D;
  const float sscale = kLog2e / sqrtf((float)D);

  using TR = TileRegs<T, D>;
  constexpr int KC = (TR::kKChunks + NT - 1) / NT;
  constexpr int VT = (TR::kVTasks + NT - 1) / NT;
  constexpr int VW = 8 * (int)sizeof(T) / 16;
  uint4 kr[KC], vr[VT * 4 * VW];
  attn_load_tile<T, D, NT>(Kb, Vb, kt0 * 64, kvalid, kr, vr);
  attn_store_tile<T, D, NT>(lds, kr, vr);
  __syncthreads();

  for (int kt = kt0; kt < kt1; ++kt) {
    const int cur = (kt - kt0) & 1;
    const bool more = kt + 1 < kt1;
    if (more) attn_load_tile<T, D, NT>(Kb, Vb, (kt + 1) * 64, kvalid, kr, vr);
    const char* kbuf = lds + cur * L::kBytes;
    const int k0 = kt * 64;

    // S^T = K Q^T: s[qb][kb] holds S[q = qb*16 + r16][key = k0 + kb*16 + 4*grp + i]
    f32x4 s[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) s[qb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const frag kf = attn_k_frag<T, D>(kbuf, kb * 16 + r16, dc, grp);
        s[0][kb] = MF::mma(kf, qf[0][dc], s[0][kb]);
        s[1][kb] = MF::mma(kf, qf[1][dc], s[1][kb]);
      }

    const bool full = (k0 + 63 <= qp_min) && (W < 0 || qp_max - k0 <= W);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qp = L0 + q0 + qb * 16 + r16;
      float mx = -INFINITY;
      if (full) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[qb][kb][i]);
      } else {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int kp = k0 + kb * 16 + 4 * grp + i;
            // bitwise, not short-circuit: a select per score instead of a branch
            const bool cut = (kp > qp) | ((W >= 0) & (qp - kp > W));
            s[qb][kb][i] = cut ? -INFINITY : s[qb][kb][i];
            mx = fmaxf(mx, s[qb][kb][i]);
          }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      // running maxima are kept on raw scores; the 1/sqrt(d) * log2(e) factor is folded
      // into the exponent: p = 2^(s c - m c)
      const float m_new = fmaxf(m_run[qb], mx);
      const float mc = m_new == -INFINITY ? 0.f : m_new * sscale;
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][kb][i], sscale, -mc));
          s[qb][kb][i] = pv;
          ps += pv;
        }
      if (__ballot(m_new != m_run[qb])) {  // some row's maximum moved: rescale
        const float alpha = __builtin_amdgcn_exp2f(m_run[qb] * sscale - mc);
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[qb][db][i] *= alpha;
      }
      l_run[qb] += ps;
      m_run[qb] = m_new;
    }

    // O^T += V^T P^T over two 32-key chunks
    const char* vt = kbuf + L::kKBytes;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      frag pf[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float pv[8] = {s[qb][2 * cc][0],     s[qb][2 * cc][1],     s[qb][2 * cc][2],     s[qb][2 * cc][3],
                             s[qb][2 * cc + 1][0], s[qb][2 * cc + 1][1], s[qb][2 * cc + 1][2], s[qb][2 * cc + 1][3]};
        pf[qb] = MF::pack(pv);
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const frag vf = load_vt_frag<T, D>(vt, db * 16 + r16, cc, grp);
        o[0][db] = MF::mma(vf, pf[0], o[0][db]);
        o[1][db] = MF::mma(vf, pf[1], o[1][db]);
      }
    }
    if (more) attn_store_tile<T, D, NT>(lds + (cur ^ 1) * L::kBytes, kr, vr);
    __syncthreads();
  }

  // lane holds O[q = qb*16 + r16][d = db*16 + 4*grp + i]; the row sum is spread over
  // the four lanes of the row
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float l = l_run[qb];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int row = qb * 16 + r16;
    const int t = q0 + row;
    if (qt.nc == 1) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      if (t < S) {
        T* orow = a.O + (((size_t)b * S + t) * a.nh + h) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          float v[4] = {o[qb][db][0] * inv, o[qb][db][1] * inv, o[qb][db][2] * inv, o[qb][db][3] * inv};
          store4(orow + db * 16 + 4 * grp, v);
        }
      }
    } else {
      float* pr = part + (((((size_t)b * a.nkv + g) * nqb + qblk) * NC + c) * G + wave) * 32 * (D + 2) +
                  (size_t)row * (D + 2);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        float v[4] = {o[qb][db][0], o[qb][db][1], o[qb][db][2], o[qb][db][3]};
        store4(pr + db * 16 + 4 * grp, v);
      }
      if (grp == 0) {  // the combine pass works in the exponent's units: m * scale
        pr[D] = m_run[qb] == -INFINITY ? -INFINITY : m_run[qb] * sscale;
        pr[D + 1] = l;
      }
    }
  }
}

// Merge the chunks of every split query tile: O = sum_c 2^(m_c - M) o_c / sum_c 2^(m_c - M) l_c.
// One thread per (query row, head, 4 dims): kRowsPerWg rows of a tile per workgroup,
// so the pass reads the partials with many independent 16-byte loads in flight.
template <int D, int G>
struct CombineShape {
  static constexpr int kNJ = D / 4;                                      // 4-dim groups per row
  static constexpr int kRowsPerWg = 256 / (G * kNJ) > 0 ? 256 / (G * kNJ) : 1;
  static constexpr int kThreads = kRowsPerWg * G * kNJ;
};

template <typename T, int D, int G, int QW = 32>
__global__ __launch_bounds__(256) void attn_prefill_combine_kernel(AttnArgs<T> a, const float* __restrict__ part,
                                                                   int NC) {
  using CS = CombineShape<D, G>;
  const int nqb = (a.S + QW - 1) / QW;
  const int qblk = blockIdx.x / (QW / CS::kRowsPerWg), g = blockIdx.y, b = blockIdx.z;
  const int L0 = cached_len(a.cache_len, b);
  const QTile qt = qtile<QW>(qblk, a.S, L0, a.window, NC);
  if (qt.nc == 1) return;
  const int j = threadIdx.x % CS::kNJ, wave = (threadIdx.x / CS::kNJ) % G;
  const int row = (blockIdx.x % (QW / CS::kRowsPerWg)) * CS::kRowsPerWg + threadIdx.x / (CS::kNJ * G);
  if (row >= qt.nq) return;
  const int h = g * G + wave;
  const size_t unit0 = (((size_t)b * a.nkv + g) * nqb + qblk) * NC;
  const size_t ustride = (size_t)G * QW * (D + 2);
  const float* base = part + (unit0 * G + wave) * QW * (D + 2) + (size_t)row * (D + 2);
  // chunks in groups of four, loads issued together (past the last chunk they re-read it).
  // The first group's maxima, sums and outputs are all requested at once, so with at most
  // four chunks the pass waits for memory once; later groups' maxima follow.
  float mc[4], lc[4];
  float4 v[4];
  auto load_group = [&](int c0) {
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const int ci = min(c0 + cc, qt.nc - 1);
      mc[cc] = base[ci * ustride + D];
      lc[cc] = base[ci * ustride + D + 1];
      v[cc] = *reinterpret_cast<const float4*>(base + ci * ustride + 4 * j);
    }
  };
  load_group(0);
  float M = fmaxf(fmaxf(mc[0], mc[1]), fmaxf(mc[2], mc[3]));
  for (int c0 = 4; c0 < qt.nc; c0 += 4) {
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) M = fmaxf(M, base[min(c0 + cc, qt.nc - 1) * ustride + D]);
  }
  float lsum = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < qt.nc; c0 += 4) {
    if (c0 > 0) load_group(c0);
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const float sc = (c0 + cc >= qt.nc || mc[cc] == -INFINITY) ? 0.f : exp2f(mc[cc] - M);
      lsum += sc * lc[cc];
      acc[0] += sc * v[cc].x;
      acc[1] += sc * v[cc].y;
      acc[2] += sc * v[cc].z;
      acc[3] += sc * v[cc].w;
    }
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  T* orow = a.O + (((size_t)b * a.S + qt.q0 + row) * a.nh + h) * D + 4 * j;
  float o4[4] = {acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
  store4(orow, o4);
}

// ----------------------------------------------------------------------------- prefill, bf16, d = 128
//
// A second prefill kernel for bf16 with head_dim 128. A unit is (64-query tile, chunk of
// its key tiles, KV group, sequence); each wave takes 32 of those queries for one query
// head of the group. QH query halves per workgroup: with 4 heads a group (the ZAYA1
// shape) a workgroup takes one half (4 waves) and two workgroups share a CU, so each
// SIMD runs two waves of different workgroups whose steps drift apart and one's softmax
// overlaps the other's products (measured 71.1 -> 68 us at 4096 tokens against one
// 8-wave workgroup per CU with both halves, whose waves met at every step's barrier);
// with 1 or 2 heads both halves share a workgroup. Both products use the 32x32x16 MFMA:
//   S^T = K Q^T  in 32-key x 32-query blocks: lane l holds query l % 32 and the keys
//                8 (r / 4) + 4 (l / 32) + r % 4, r < 16, of the block;
//   O^T = V^T P^T in 32-dim x 32-query blocks over 16-key steps: the B operand of step
//                ks is eight of the lane's score registers as they are (registers
//                8 (ks % 2) .. +8 of key block ks / 2: keys 16 ks + 4 (l / 32) + 0..3 and
//                16 ks + 8 + 4 (l / 32) + 0..3), and the A operand holds the V values of
//                the same keys for dim l % 32 of the block.
// K and V tiles go from global memory straight into LDS (global_load_lds, row-major
// [key][dim], a 16-byte-chunk swizzle applied on the global side) through a ring of LDS
// slots declared as separate arrays (so the compiler's wait tracking sees that the loads
// into one slot cannot alias reads of another): two slots, one tile ahead of the
// products, so two workgroups fit a CU (three slots, two tiles ahead, serve an 8-wave
// workgroup alone on its CU). The V^T operands come from the row-major V tile through the LDS transpose
// read (ds_read_b64_tr_b16): within each 16-lane group, lane a + 4 k addresses 4 dims
// of key row k and lane 4 a + c receives dim c of that chunk for the 4 keys. Each wave
// waits only for the tile the next step reads (the newest tile's loads stay in flight)
// and the workgroup then meets at a bare barrier. The loop is unrolled by three, so every
// fragment read is a per-lane offset (computed once) plus an immediate.
namespace pf64 {
constexpr int kQW = 64;                  // queries per workgroup (per head)
constexpr int kD = 128;
constexpr int kRow = kD * 2;             // bytes per K or V row (bf16)
constexpr int kTileBytes = 64 * kRow;    // one 64-key K or V tile
constexpr int kBuf = 2 * kTileBytes;     // a slot: K tile, then V tile
// Measured on gfx950 for these fragment reads (32 key rows of one 16-byte chunk per
// half wave): chunk c of key k stored at c ^ (k % 16) reads conflict-free (118 TB/s);
// the swizzle of the 16x16 kernel drops to 69 TB/s here.
__device__ __forceinline__ int koff(int key, int chunk) { return key * kRow + ((chunk ^ (key & 15)) << 4); }
// V: chunk c of key k stored at c ^ vsw(k). A transpose read covers 8 consecutive keys
// (a multiple of 8 onwards) x 32 bytes of one 64-byte dim block per 16-lane group, 512
// bytes per wave: with 128 four-byte banks a key row spans half of them (even and odd
// keys on opposite halves), and vsw puts the 64-byte blocks of the four keys of each
// half in four different places.
__device__ __forceinline__ int vsw(int key) { return ((key >> 1) & 3) << 2; }
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x16 mma(const uint4& a, const uint4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}
__device__ __forceinline__ uint2 read_tr(const char* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(__attribute__((address_space(3))) const char*)(p));
  return __builtin_bit_cast(uint2, v);
}
// s_waitcnt immediate that waits until at most n vector memory operations are pending
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
}  // namespace pf64

template <int G, int QH>
__global__ __launch_bounds__(64 * QH * G) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_prefill64_kernel(
    AttnArgs<bf16_t> a, float* __restrict__ part, int NC) {
  using namespace pf64;
  constexpr int NW = QH * G;                          // waves
  constexpr int NSLOT = (G == 4 && QH == 2) ? 3 : 2;  // ring slots; tiles in flight ahead: NSLOT - 1
  constexpr int kLoads = 16 / NW;  // 16-byte load instructions per thread per K (or V) tile
  constexpr int kTileLoads = 2 * kLoads;   // per thread per tile (K and V)
  constexpr int kPendOk = (NSLOT - 2) * kTileLoads;  // loads that may stay in flight at a step's end
  static_assert(NW * kLoads * 4 == 64, "one tile: 64 rows of 4 per instruction");
  __shared__ __attribute__((aligned(1024))) char lds0[kBuf];
  __shared__ __attribute__((aligned(1024))) char lds1[kBuf];
  __shared__ __attribute__((aligned(1024))) char lds2[NSLOT == 3 ? kBuf : 16];

  // units heaviest first over the whole grid: (query tile from the last, chunk, query
  // half when a workgroup takes one), then KV group and sequence fastest, so the longest
  // units of every group and sequence start in the first round
  const int nqb = (a.S + kQW - 1) / kQW;
  const int ngb = a.nkv * a.B;
  const int gb = (int)blockIdx.x % ngb;
  const int r = QH == 2 ? (int)blockIdx.x / ngb : (int)blockIdx.x / ngb / 2;
  const int half = QH == 2 ? 0 : ((int)blockIdx.x / ngb) % 2;
  const int c = r % NC;
  const int qblk = nqb - 1 - r / NC;
  const int g = gb % a.nkv, b = gb / a.nkv;
  const int S = a.S, L0 = cached_len(a.cache_len, b), W = a.window;
  const QTile qt = qtile<kQW>(qblk, S, L0, W, NC);
  if (c >= qt.nc) return;
  const int kt0 = qt.kt_begin + c * qt.n / qt.nc;
  const int kt1 = qt.kt_begin + (c + 1) * qt.n / qt.nc;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hl = lane >> 5;
  const int hg = wave % G, qh = QH == 2 ? wave / G : half;  // head within the group, query half
  const int h = g * G + hg;
  const int row = qh * 32 + l32;           // this lane's query within the tile
  const int q0 = qt.q0, qp_min = qt.qp_min, qp_max = qt.qp_max;
  const int qp = L0 + q0 + row;
  const int kvalid = L0 + S;
  const bf16_t* Kb = a.K + ((size_t)b * a.nkv + g) * a.cap * kD;
  const bf16_t* Vb = a.V + ((size_t)b * a.nkv + g) * a.cap * kD;
  const float sscale = kLog2e / sqrtf((float)kD);

  // Tile loads: instruction j of a wave fills key rows kr0 .. kr0 + 3 (1 KiB, 16 bytes a
  // lane, in LDS order); the lane at position p of its row fetches the chunk stored
  // there. Key rows past kvalid - 1 re-read that row: those keys come after every query
  // of the call, so their scores are masked and their probabilities are exactly 0; tiles
  // past the unit's range re-read valid rows into a slot nothing reads.
  auto issue_tile = [&](char* buf, int k0) {
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int kr0 = (wave * kLoads + j) * 4;
      const int key = kr0 + (lane >> 4);
      const bf16_t* src = Kb + (size_t)min(k0 + key, kvalid - 1) * kD + (((lane & 15) ^ (key & 15)) << 3);
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(buf + kr0 * kRow), 16, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int kr0 = (wave * kLoads + j) * 4;
      const int key = kr0 + (lane >> 4);
      const bf16_t* src = Vb + (size_t)min(k0 + key, kvalid - 1) * kD + (((lane & 15) ^ vsw(key)) << 3);
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(buf + kTileBytes + kr0 * kRow), 16,
                                       0, 0);
    }
  };
  // this lane's query (zero past S): dims 16 ds + 8 hl .. + 8; then the first tiles
  uint4 qf[8];
  {
    const int t = q0 + row;
    const bf16_t* qrow = a.Q + (((size_t)b * S + min(t, S - 1)) * a.nh + h) * kD + 8 * hl;
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) {
      const uint4 v = *reinterpret_cast<const uint4*>(qrow + 16 * ds);
      qf[ds] = t < S ? v : make_uint4(0, 0, 0, 0);
    }
  }
  issue_tile(lds0, kt0 * 64);
  if constexpr (NSLOT == 3) issue_tile(lds1, (kt0 + 1) * 64);
  // fragment offsets within a slot: K for step ds (key block 0; block 1 is 32 rows on);
  // V for dim block db (PV step ks and its second four keys: immediates on top). A lane
  // of 16-lane group gi = lane / 16 at position i reads key row 4 hl + i / 4 (+ 16 ks,
  // + 8), dims 32 db + 16 (gi % 2) + 4 (i % 4) .. + 3.
  int ko[8], vo[4];
#pragma unroll
  for (int ds = 0; ds < 8; ++ds) ko[ds] = koff(l32, 2 * ds + hl);
  {
    const int i = lane & 15, gi = lane >> 4;
    const int vkey = 4 * hl + (i >> 2);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int byte = 64 * db + 32 * (gi & 1) + 8 * (i & 3);
      vo[db] = kTileBytes + vkey * kRow + ((((byte >> 4) ^ vsw(vkey))) << 4) + (byte & 15);
    }
  }

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // One key tile j in ring slot B; tile j + NSLOT - 1 loads into the slot before it.
  auto step = [&](auto slot_tag, int j) {
    constexpr int B = decltype(slot_tag)::value;
    constexpr int BA = (B + NSLOT - 1) % NSLOT;
    const char* buf = B == 0 ? lds0 : (B == 1 ? lds1 : lds2);
    char* ahead = BA == 0 ? lds0 : (BA == 1 ? lds1 : lds2);
    issue_tile(ahead, (j + NSLOT - 1) * 64);
    const int k0 = j * 64;
    // S^T = K Q^T
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
    for (int ds = 0; ds < 8; ++ds)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint4 kf = *reinterpret_cast<const uint4*>(buf + ko[ds] + kb * 32 * kRow);
        s[kb] = mma(kf, qf[ds], s[kb]);
      }
    // mask where the tile cuts the causal / window band; running max; rescale
    const bool full = (k0 + 63 <= qp_min) && (W < 0 || qp_max - k0 <= W);
    if (!full) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kp = k0 + kb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
          // bitwise, not short-circuit: a select per score instead of a branch
          const bool cut = (kp > qp) | ((W >= 0) & (qp - kp > W));
          s[kb][r] = cut ? -INFINITY : s[kb][r];
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float mc = m_new == -INFINITY ? 0.f : m_new * sscale;
    if (__ballot(m_new != m_run)) {  // some row's maximum moved: rescale
      const float alpha = __builtin_amdgcn_exp2f(m_run * sscale - mc);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    }
    m_run = m_new;
    // probabilities (exponent base 2, the 1/sqrt(d) log2(e) factor folded in), row sum,
    // bf16 B fragments
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], sscale, -mc));
        s[kb][r] = pv;
        ps += pv;
      }
    l_run += ps;
    uint4 pf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kb = ks >> 1, r0 = 8 * (ks & 1);
      pf[ks] = make_uint4(pack_bf16x2(s[kb][r0], s[kb][r0 + 1]), pack_bf16x2(s[kb][r0 + 2], s[kb][r0 + 3]),
                          pack_bf16x2(s[kb][r0 + 4], s[kb][r0 + 5]), pack_bf16x2(s[kb][r0 + 6], s[kb][r0 + 7]));
    }
    // O^T += V^T P^T
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const uint2 lo = read_tr(buf + vo[db] + 16 * ks * kRow);
        const uint2 hi = read_tr(buf + vo[db] + (16 * ks + 8) * kRow);
        o[db] = mma(make_uint4(lo.x, lo.y, hi.x, hi.y), pf[ks], o[db]);
      }
    // tile j + 1 has landed for this wave (with three slots tile j + 2's loads, the
    // youngest, stay in flight); after the barrier every wave's part of it has
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kPendOk));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  using Slot0 = std::integral_constant<int, 0>;
  using Slot1 = std::integral_constant<int, 1>;
  using Slot2 = std::integral_constant<int, 2>;

  // the queries and tile kt0 have landed (with three slots tile kt0 + 1 may be in flight)
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(kPendOk));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  // whole rounds of the ring first (no branch inside, so the compiler's wait tracking
  // sees the same loads in flight on every path back to the loop's head), then the rest
  int j = kt0;
  for (; j + NSLOT <= kt1; j += NSLOT) {
    step(Slot0{}, j);
    step(Slot1{}, j + 1);
    if constexpr (NSLOT == 3) step(Slot2{}, j + 2);
  }
  if (j < kt1) step(Slot0{}, j);
  if constexpr (NSLOT == 3)
    if (j + 1 < kt1) step(Slot1{}, j + 1);
  // no load may still be writing LDS when the workgroup ends
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  // lane holds O^T[d = 32 db + 8 (r / 4) + 4 hl + r % 4][its query]; the row sum is
  // split over lanes l32 and l32 + 32
  const float l = l_run + __shfl_xor(l_run, 32, 64);
  const int t = q0 + row;
  if (qt.nc == 1) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (t < S) {
      bf16_t* orow = a.O + (((size_t)b * S + t) * a.nh + h) * kD;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          float v[4] = {o[db][4 * gq] * inv, o[db][4 * gq + 1] * inv, o[db][4 * gq + 2] * inv,
                        o[db][4 * gq + 3] * inv};
          store4(orow + db * 32 + 8 * gq + 4 * hl, v);
        }
    }
  } else {
    float* pr = part + (((((size_t)b * a.nkv + g) * nqb + qblk) * NC + c) * G + hg) * kQW * (kD + 2) +
                (size_t)row * (kD + 2);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        float v[4] = {o[db][4 * gq], o[db][4 * gq + 1], o[db][4 * gq + 2], o[db][4 * gq + 3]};
        store4(pr + db * 32 + 8 * gq + 4 * hl, v);
      }
    if (hl == 0) {  // the combine pass works in the exponent's units: m * scale
      pr[kD] = m_run == -INFINITY ? -INFINITY : m_run * sscale;
      pr[kD + 1] = l;
    }
  }
}

// ----------------------------------------------------------------------------- decode

constexpr int kDecChunkMin = 256;   // keys per decode chunk, at least
constexpr int kDecChunksMax = 128;  // chunks per (sequence, KV group), at most

template <typename T, int D, int G>
__global__ __launch_bounds__(64 * G) void attn_decode_kernel(AttnArgs<T> a, float* __restrict__ part, int nchunk) {
  constexpr int NT = 64 * G;
  constexpr int KROW = D * (int)sizeof(T) + 16;
  constexpr int VROW = D * (int)sizeof(T) + 16;
  constexpr int DPL = D / 64;  // dims per lane in the weighted sum
  __shared__ __attribute__((aligned(16))) char kt_s[64 * KROW];
  __shared__ __attribute__((aligned(16))) char vt_s[64 * VROW];
  __shared__ __attribute__((aligned(16))) float q_s[G][D];
  __shared__ __attribute__((aligned(16))) float p_s[G][64];
  // bf16: the query as stored and the probabilities rounded to bf16, for the
  // v_dot2_f32_bf16 products (each multiplies two bf16 pairs exactly, sums in fp32)
  constexpr bool kDot2 = sizeof(T) == 2;
  __shared__ __attribute__((aligned(16))) uint32_t q2_s[G][D / 2];
  __shared__ __attribute__((aligned(16))) uint32_t p2_s[G][32];

  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = g * G + wave;
  const int L0 = cached_len(a.cache_len, b);
  const int qp = L0;  // the new token's position
  // a linear cache holds positions below cap only (a position past it was not stored)
  const int kvalid = a.ring ? L0 + 1 : min(L0 + 1, a.cap);
  const int W = a.window;
  const int klo = W >= 0 ? max(0, qp - W) : 0;
  // the nchunk chunks of this sequence tile its visible range from the 64-aligned
  // position at or below its start; the chunk length follows from the sequence's own
  // cache length on the device, so the grid covers every key whatever that length is
  const int kbase = (klo / 64) * 64;
  const int span = max(kvalid - kbase, 1);
  const int chunk = ((span + nchunk - 1) / nchunk + 63) / 64 * 64;
  const int c_lo = max(klo, kbase + c * chunk), c_hi = min(kvalid, kbase + (c + 1) * chunk);
  const float sscale = kLog2e / sqrtf((float)D);

  if constexpr (kDot2) {
    const uint32_t* qg = reinterpret_cast<const uint32_t*>(a.Q + ((size_t)b * a.nh + h) * D);
    for (int i = lane; i < D / 2; i += 64) q2_s[wave][i] = qg[i];
  } else {
    for (int i = lane; i < D; i += 64) q_s[wave][i] = Act<T>::tof(a.Q[((size_t)b * a.nh + h) * D + i]);
  }

  float m_run = -INFINITY, l_run = 0.f;
  float o[DPL];
#pragma unroll
  for (int j = 0; j < DPL; ++j) o[j] = 0.f;

  const T* Kb = a.K + ((size_t)b * a.nkv + g) * a.cap * D;
  const T* Vb = a.V + ((size_t)b * a.nkv + g) * a.cap * D;
  constexpr int E16 = 16 / (int)sizeof(T);
  constexpr int CPR = D / E16;               // 16-byte chunks per row
  constexpr int NCH = 64 * CPR;              // per tile, per tensor
  constexpr int PER = (NCH + NT - 1) / NT;
  uint4 kr[PER], vr[PER];
  auto load = [&](int t0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int ch = threadIdx.x + i * NT;
      const int key = ch / CPR, col = (ch % CPR) * E16;
      const bool ok = ch < NCH && t0 + key < c_hi;
      const size_t slot = a.ring ? (size_t)((t0 + key) % a.cap) : (size_t)(t0 + key);  // ring: p % cap
      // the cache is streamed once per step: non-temporal loads keep it out of the caches
      const u32x4 kq = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Kb + slot * D + col))
                          : u32x4{0u, 0u, 0u, 0u};
      const u32x4 vq = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Vb + slot * D + col))
                          : u32x4{0u, 0u, 0u, 0u};
      kr[i] = make_uint4(kq[0], kq[1], kq[2], kq[3]);
      vr[i] = make_uint4(vq[0], vq[1], vq[2], vq[3]);
    }
  };
  const int t_first = (c_lo / 64) * 64;
  if (t_first < c_hi) load(t_first);
  for (int t0 = t_first; t0 < c_hi; t0 += 64) {
    __syncthreads();  // previous tile consumed (and q_s written on the first pass)
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int ch = threadIdx.x + i * NT;
      if (ch < NCH) {
        const int key = ch / CPR, colb = (ch % CPR) * 16;
        *reinterpret_cast<uint4*>(kt_s + key * KROW + colb) = kr[i];
        *reinterpret_cast<uint4*>(vt_s + key * VROW + colb) = vr[i];
      }
    }
    __syncthreads();
    if (t0 + 64 < c_hi) load(t0 + 64);  // next tile in flight during this one
    // scores: lane = key
    const int kp = t0 + lane;
    const T* krow = reinterpret_cast<const T*>(kt_s + lane * KROW);
    float acc0 = 0.f, acc1 = 0.f;
    if constexpr (kDot2) {
#pragma unroll
      for (int i = 0; i < D; i += 8) {
        const u32x4 kv = *reinterpret_cast<const u32x4*>(krow + i);
        const u32x4 qv = *reinterpret_cast<const u32x4*>(&q2_s[wave][i / 2]);
        acc0 = dot2_bf16(kv[0], qv[0], acc0);
        acc1 = dot2_bf16(kv[1], qv[1], acc1);
        acc0 = dot2_bf16(kv[2], qv[2], acc0);
        acc1 = dot2_bf16(kv[3], qv[3], acc1);
      }
    } else {
#pragma unroll
      for (int i = 0; i < D; i += 8) {
        float kv[8];
        load4(krow + i, kv);
        load4(krow + i + 4, kv + 4);
        const float4 qa = *reinterpret_cast<const float4*>(&q_s[wave][i]);
        const float4 qb = *reinterpret_cast<const float4*>(&q_s[wave][i + 4]);
        acc0 += qa.x * kv[0] + qa.y * kv[1] + qa.z * kv[2] + qa.w * kv[3];
        acc1 += qb.x * kv[4] + qb.y * kv[5] + qb.z * kv[6] + qb.w * kv[7];
      }
    }
    const bool vis = kp >= c_lo && kp < c_hi;
    const float sv = vis ? (acc0 + acc1) * sscale : -INFINITY;
    const float mx = wave_max(sv);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    const float pv = __builtin_amdgcn_exp2f(sv - m_use);
    l_run = l_run * alpha + pv;
    m_run = m_new;
    if constexpr (kDot2) {
      // key pairs (2m, 2m+1): the lane of key 2m packs both probabilities
      const float pnext = dpp_mov<0xF5>(pv);  // quad_perm [1, 1, 3, 3]: lane 2m reads lane 2m + 1
      if (!(lane & 1)) p2_s[wave][lane >> 1] = pack_bf16x2(pv, pnext);
    } else {
      p_s[wave][lane] = pv;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int j = 0; j < DPL; ++j) o[j] *= alpha;
    // weighted sum: lane owns dims [lane*DPL, lane*DPL + DPL)
    if constexpr (kDot2 && DPL == 2) {
      // two keys per product: (v_k[d], v_k+1[d]) pairs built with one byte permute each
#pragma unroll 4
      for (int k = 0; k < 64; k += 8) {
        const u32x4 pp = *reinterpret_cast<const u32x4*>(&p2_s[wave][k / 2]);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const uint32_t v0 = *reinterpret_cast<const uint32_t*>(vt_s + (k + 2 * kk) * VROW + lane * 4);
          const uint32_t v1 = *reinterpret_cast<const uint32_t*>(vt_s + (k + 2 * kk + 1) * VROW + lane * 4);
          o[0] = dot2_bf16(pp[kk], __builtin_amdgcn_perm(v1, v0, 0x05040100u), o[0]);  // low halves: dim 2 lane
          o[1] = dot2_bf16(pp[kk], __builtin_amdgcn_perm(v1, v0, 0x07060302u), o[1]);  // high halves
        }
      }
    } else if constexpr (kDot2) {
      // head_dim 64: one dim per lane, two keys per product (v_k[lane], v_k+1[lane])
#pragma unroll 4
      for (int k = 0; k < 64; k += 8) {
        const u32x4 pp = *reinterpret_cast<const u32x4*>(&p2_s[wave][k / 2]);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const uint32_t v0 = *reinterpret_cast<const uint16_t*>(vt_s + (k + 2 * kk) * VROW + lane * 2);
          const uint32_t v1 = *reinterpret_cast<const uint16_t*>(vt_s + (k + 2 * kk + 1) * VROW + lane * 2);
          o[0] = dot2_bf16(pp[kk], v0 | (v1 << 16), o[0]);
        }
      }
    } else {
      // four keys per step
#pragma unroll 4
      for (int k = 0; k < 64; k += 4) {
        const float4 pk = *reinterpret_cast<const float4*>(&p_s[wave][k]);
        const float pkk[4] = {pk.x, pk.y, pk.z, pk.w};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const T* vrow = reinterpret_cast<const T*>(vt_s + (k + kk) * VROW) + lane * DPL;
#pragma unroll
          for (int j = 0; j < DPL; ++j) o[j] += pkk[kk] * Act<T>::tof(vrow[j]);
        }
      }
    }
  }
  l_run = wave_sum(l_run);
  float* pp = part + ((((size_t)b * a.nkv + g) * nchunk + c) * G + wave) * (D + 2);
#pragma unroll
  for (int j = 0; j < DPL; ++j) pp[lane * DPL + j] = o[j];
  if (lane == 0) {
    pp[D] = m_run;
    pp[D + 1] = l_run;
  }
}

// Merge the key chunks of one (sequence, head): each lane owns D/64 dims; the chunk
// maxima are read in one pass so all loads are independent.
template <typename T, int D, int G>
__global__ __launch_bounds__(64) void attn_decode_combine_kernel(AttnArgs<T> a, const float* __restrict__ part,
                                                                  int nchunk) {
  const int bh = blockIdx.x;
  const int b = bh / a.nh, h = bh % a.nh;
  const int g = h / G, w = h % G;
  const float* base = part + (((size_t)b * a.nkv + g) * nchunk * G + w) * (D + 2);
  const size_t stride = (size_t)G * (D + 2);
  constexpr int DPL = D / 64;  // dims per lane
  constexpr int kBatch = 32;   // chunks whose partial outputs are requested at once
  __shared__ float sc_s[kDecChunksMax];
  // every load the merge needs before its first use: the chunk maxima and sums of this
  // lane's chunks (c = lane, lane + 64) and the first kBatch chunks' outputs
  float m2[2], l2[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = (int)threadIdx.x + 64 * k;
    m2[k] = c < nchunk ? base[c * stride + D] : -INFINITY;
    l2[k] = c < nchunk ? base[c * stride + D + 1] : 0.f;
  }
  const float* pl = base + threadIdx.x * DPL;
  float ov[kBatch][DPL];
#pragma unroll
  for (int c = 0; c < kBatch; ++c)
#pragma unroll
    for (int j = 0; j < DPL; ++j) ov[c][j] = c < nchunk ? pl[c * stride + j] : 0.f;
  const float M = wave_max(fmaxf(m2[0], m2[1]));
  float lpart = 0.f;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = (int)threadIdx.x + 64 * k;
    if (c < nchunk) {
      const float sc = m2[k] == -INFINITY ? 0.f : exp2f(m2[k] - M);
      sc_s[c] = sc;
      lpart += sc * l2[k];
    }
  }
  const float L = wave_sum(lpart);
  __syncthreads();
  float acc[DPL];
#pragma unroll
  for (int j = 0; j < DPL; ++j) acc[j] = 0.f;
#pragma unroll
  for (int c = 0; c < kBatch; ++c)
    if (c < nchunk)
#pragma unroll
      for (int j = 0; j < DPL; ++j) acc[j] += sc_s[c] * ov[c][j];
  for (int c0 = kBatch; c0 < nchunk; c0 += kBatch) {  // further chunks, kBatch loads at a time
#pragma unroll
    for (int c = 0; c < kBatch; ++c)
#pragma unroll
      for (int j = 0; j < DPL; ++j) ov[c][j] = c0 + c < nchunk ? pl[(c0 + c) * stride + j] : 0.f;
#pragma unroll
    for (int c = 0; c < kBatch; ++c)
      if (c0 + c < nchunk)
#pragma unroll
        for (int j = 0; j < DPL; ++j) acc[j] += sc_s[c0 + c] * ov[c][j];
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  T* orow = a.O + ((size_t)b * a.nh + h) * D;
#pragma unroll
  for (int j = 0; j < D / 64; ++j) orow[threadIdx.x * (D / 64) + j] = Act<T>::cvt(acc[j] * inv);
}

template <typename T, int D, int G>
static hipError_t launch_prefill_dg(const AttnArgs<T>& a, float* part, int NC, hipStream_t s) {
  if constexpr (sizeof(T) == 2 && D == 128 && G <= 4) {
    const int nqb = (a.S + pf64::kQW - 1) / pf64::kQW;
    constexpr int QH = G == 4 ? 1 : 2;  // query halves per workgroup
    hipLaunchKernelGGL((attn_prefill64_kernel<G, QH>), dim3(nqb * NC * a.nkv * a.B * (2 / QH)), dim3(64 * QH * G), 0,
                       s, a, part, NC);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || NC == 1) return e;
    using CS = CombineShape<D, G>;
    hipLaunchKernelGGL((attn_prefill_combine_kernel<T, D, G, pf64::kQW>),
                       dim3(nqb * (pf64::kQW / CS::kRowsPerWg), a.nkv, a.B), dim3(CS::kThreads), 0, s, a, part, NC);
    return hipGetLastError();
  }
  const int nqb = (a.S + 31) / 32;
  hipLaunchKernelGGL((attn_prefill_kernel<T, D, G>), dim3(nqb * NC, a.nkv, a.B), dim3(64 * G), 0, s, a, part, NC);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || NC == 1) return e;
  using CS = CombineShape<D, G>;
  hipLaunchKernelGGL((attn_prefill_combine_kernel<T, D, G>), dim3(nqb * (32 / CS::kRowsPerWg), a.nkv, a.B),
                     dim3(CS::kThreads), 0, s, a, part, NC);
  return hipGetLastError();
}

template <typename T, int D, int G>
static hipError_t launch_decode_dg(const AttnArgs<T>& a, float* part, int span, hipStream_t s) {
  // chunk count from the host's largest span; each sequence's chunk length is derived
  // on the device (the kernel), so a call replayed with grown cache lengths (a captured
  // graph) still visits every key, in fewer, longer chunks
  int nchunk = min(kDecChunksMax, (span + kDecChunkMin - 1) / kDecChunkMin);
  const int chunk = (((span + nchunk - 1) / nchunk) + 63) / 64 * 64;
  nchunk = (span + chunk - 1) / chunk;
  hipLaunchKernelGGL((attn_decode_kernel<T, D, G>), dim3(nchunk, a.nkv, a.B), dim3(64 * G), 0, s, a, part, nchunk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_decode_combine_kernel<T, D, G>), dim3(a.B * a.nh), dim3(64), 0, s, a, part, nchunk);
  return hipGetLastError();
}

#define ZAYA_DISPATCH_DG(FN, ...)                                 \
  do {                                                            \
    const int G_ = a.nh / a.nkv;                                  \
    if (a.d == 128) {                                             \
      if (G_ == 1) return FN<T, 128, 1>(__VA_ARGS__);             \
      if (G_ == 2) return FN<T, 128, 2>(__VA_ARGS__);             \
      if (G_ == 4) return FN<T, 128, 4>(__VA_ARGS__);             \
      if (G_ == 8) return FN<T, 128, 8>(__VA_ARGS__);             \
    } else if (a.d == 64) {                                       \
      if (G_ == 1) return FN<T, 64, 1>(__VA_ARGS__);              \
      if (G_ == 2) return FN<T, 64, 2>(__VA_ARGS__);              \
      if (G_ == 4) return FN<T, 64, 4>(__VA_ARGS__);              \
      if (G_ == 8) return FN<T, 64, 8>(__VA_ARGS__);              \
    }                                                             \
    return hipErrorInvalidValue;                                  \
  } while (0)

template <typename T>
hipError_t launch_attn_prefill(const AttnArgs<T>& a, float* part, int NC, hipStream_t s) {
  ZAYA_DISPATCH_DG(launch_prefill_dg, a, part, NC, s);
}

int attn_prefill_chunk_tiles(int act_bytes, int d, int G) {
  return act_bytes == 2 && d == 128 && G <= 4 ? kPrefill64ChunkTiles : kPrefillChunkTiles;
}

// Chunks per query tile: enough that no unit exceeds chunk_tiles key tiles of the
// longest query tile (capped at 16).
int attn_prefill_chunks(int S, int max_cache_len, int window, int chunk_tiles) {
  const int qp_max = max_cache_len + S - 1;
  const int klo = window >= 0 ? (qp_max - 31 - window > 0 ? qp_max - 31 - window : 0) : 0;
  const int tiles = qp_max / 64 + 1 - klo / 64;
  int nc = (tiles + chunk_tiles - 1) / chunk_tiles;
  return nc < 1 ? 1 : (nc > 16 ? 16 : nc);
}

// Sized for 64-query tiles, which covers the 32-query tiles of the other kernel too.
size_t attn_prefill_part_bytes(int B, int S, int nkv, int G, int d, int NC) {
  if (NC <= 1) return 0;
  const size_t rows = (size_t)(S + 63) / 64 * 64;
  return (size_t)B * nkv * rows * NC * G * (d + 2) * sizeof(float);
}

template <typename T>
hipError_t launch_attn_decode(const AttnArgs<T>& a, float* part, int span, hipStream_t s) {
  ZAYA_DISPATCH_DG(launch_decode_dg, a, part, span, s);
}

size_t attn_decode_part_bytes(int B, int nkv, int G, int d) {
  return (size_t)B * nkv * kDecChunksMax * G * (d + 2) * sizeof(float);
}

template hipError_t launch_attn_prefill<bf16_t>(const AttnArgs<bf16_t>&, float*, int, hipStream_t);
template hipError_t launch_attn_prefill<float>(const AttnArgs<float>&, float*, int, hipStream_t);
template hipError_t launch_attn_decode<bf16_t>(const AttnArgs<bf16_t>&, float*, int, hipStream_t);
template hipError_t launch_attn_decode<float>(const AttnArgs<float>&, float*, int, hipStream_t);

}  // namespace zaya
