// Stream RMSNorm and the embedding gather (HBM-bound; one wave per row).
//
// ZayaRMSNorm on the float32 stream ("The stream is float32 whatever the load" on the
// nnterp page: the norm casts the stream to the weight dtype first, then norms it):
//   xa = rnd(x);  y = rnd(xa / sqrt(mean(xa^2) + eps));  out = rnd(g * y)
// Embedding ("The stream is float32 whatever the load": shift and scale, then the
// cast to float32):  x0 = f32(rnd(rnd(E[id] + shift) * scale)).
#include "common.h"
#include "kernels.h"

namespace zaya {

// rows: number of rows; H % 256 == 0. Each lane owns H/256 groups of 4 consecutive
// columns, strided 256 apart, so every wave-wide load is contiguous.
template <typename T, int NG>
__global__ __launch_bounds__(256) void rmsnorm_stream_kernel(const float* __restrict__ x, const T* __restrict__ g,
                                                               T* __restrict__ out, int rows, int H, float eps) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float* xr = x + (size_t)row * H;
  T* orow = out + (size_t)row * H;
  constexpr int kMaxGroups = NG;  // H / 256 (compile time: registers for exactly this row)
  float v[kMaxGroups][4], gv[kMaxGroups][4];
  const int ng = NG;
  // the row and the gain are requested together: one memory round trip per row
#pragma unroll
  for (int i = 0; i < kMaxGroups; ++i)
    if (i < ng) {
      load4(xr + i * 256 + lane * 4, v[i]);
      load4(g + i * 256 + lane * 4, gv[i]);
    }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxGroups; ++i) {
    if (i < ng) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        v[i][c] = Act<T>::rnd(v[i][c]);
        ss += v[i][c] * v[i][c];
      }
    }
  }
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)H + eps);
#pragma unroll
  for (int i = 0; i < kMaxGroups; ++i) {
    if (i < ng) {
      float o[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) o[c] = Act<T>::rnd(gv[i][c] * Act<T>::rnd(v[i][c] * inv));
      store4(orow + i * 256 + lane * 4, o);
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ ids, const T* __restrict__ table,
                                                      const T* __restrict__ shift, const T* __restrict__ scale,
                                                      float* __restrict__ x0, T* __restrict__ tap, int rows, int H,
                                                      int vocab) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  int id = ids[row];
  if (id < 0 || id >= vocab) id = 0;
  const T* er = table + (size_t)id * H;
  for (int c0 = lane * 4; c0 < H; c0 += 256) {
    float e[4], sh[4], sc[4], o[4];
    load4(er + c0, e);
    load4(shift + c0, sh);
    load4(scale + c0, sc);
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] = Act<T>::rnd(Act<T>::rnd(e[c] + sh[c]) * sc[c]);
    store4(x0 + (size_t)row * H + c0, o);
    if (tap) store4(tap + (size_t)row * H + c0, o);
  }
}

template <typename T>
hipError_t launch_rmsnorm_stream(const float* x, const T* g, T* out, int rows, int H, float eps, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const dim3 grid((rows + 3) / 4), block(256);
  switch (H / 256) {  // H is a multiple of 256, at most 4096 (checked by the host)
#define ZAYA_NORM_CASE(n) \
  case n: hipLaunchKernelGGL((rmsnorm_stream_kernel<T, n>), grid, block, 0, s, x, g, out, rows, H, eps); break;
    ZAYA_NORM_CASE(1) ZAYA_NORM_CASE(2) ZAYA_NORM_CASE(3) ZAYA_NORM_CASE(4) ZAYA_NORM_CASE(5) ZAYA_NORM_CASE(6)
    ZAYA_NORM_CASE(7) ZAYA_NORM_CASE(8) ZAYA_NORM_CASE(9) ZAYA_NORM_CASE(10) ZAYA_NORM_CASE(11) ZAYA_NORM_CASE(12)
    ZAYA_NORM_CASE(13) ZAYA_NORM_CASE(14) ZAYA_NORM_CASE(15) ZAYA_NORM_CASE(16)
#undef ZAYA_NORM_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Decode tail of the attention half, one workgroup per row (few rows, so the row is
// spread over 256 threads): o = rnd(sum of the split-K partials, in part order), the
// attention merge exactly as the o_proj merge epilogue (attention_output =
// rnd(rnd(o + hsb) * hss); h = f32(f32(x + rb) * rs) + attention_output), then the
// post-attention RMSNorm of h as rmsnorm_stream_kernel computes it (the sum of squares
// reduced over the workgroup). Thread t owns columns 4t + 1024 i .. +3, i < NG = H / 1024
// rounded up. Every load is issued before the first is used: the row's stream values,
// the merge vectors and the norm gain, then the partials, eight parts at a time.
template <typename T, int NG>
__global__ __launch_bounds__(256) void merge_norm_parts_kernel(const float* __restrict__ part, int kparts, int rows,
                                                               int H, const float* __restrict__ x,
                                                               const T* __restrict__ hsb, const T* __restrict__ hss,
                                                               const T* __restrict__ rb, const T* __restrict__ rs,
                                                               float* __restrict__ h, T* __restrict__ a_tap,
                                                               const T* __restrict__ g2, T* __restrict__ hn,
                                                               float eps) {
  __shared__ float red[4];
  const int row = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float o[NG][4], xs[NG][4], b1[NG][4], s1[NG][4], b2[NG][4], s2[NG][4], gv[NG][4];
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    const int n = min((int)threadIdx.x * 4 + i * 1024, H - 4);  // clamped: columns past H are never stored
#pragma unroll
    for (int c = 0; c < 4; ++c) o[i][c] = 0.f;
    load4(x + (size_t)row * H + n, xs[i]);
    load4(hsb + n, b1[i]);
    load4(hss + n, s1[i]);
    load4(rb + n, b2[i]);
    load4(rs + n, s2[i]);
    load4(g2 + n, gv[i]);
  }
  for (int k0 = 0; k0 < kparts; k0 += 8) {  // summed in part order from zero
    float w[8][NG][4];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (k0 + k < kparts)
#pragma unroll
        for (int i = 0; i < NG; ++i)
          load4(part + ((size_t)(k0 + k) * rows + row) * H + min((int)threadIdx.x * 4 + i * 1024, H - 4), w[k][i]);
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (k0 + k < kparts)
#pragma unroll
        for (int i = 0; i < NG; ++i)
#pragma unroll
          for (int c = 0; c < 4; ++c) o[i][c] += w[k][i][c];
  }
  float v[NG][4];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    const int n = (int)threadIdx.x * 4 + i * 1024;
    float at[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float oc = Act<T>::rnd(o[i][c]);
      at[c] = Act<T>::rnd(Act<T>::rnd(oc + b1[i][c]) * s1[i][c]);
      v[i][c] = fadd(fmul(fadd(xs[i][c], b2[i][c]), s2[i][c]), at[c]);
    }
    if (n < H) {
      store4(h + (size_t)row * H + n, v[i]);
      if (a_tap) store4(a_tap + (size_t)row * H + n, at);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        v[i][c] = Act<T>::rnd(v[i][c]);
        ss += v[i][c] * v[i][c];
      }
    }
  }
  ss = wave_sum(ss);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  ss = red[0] + red[1] + red[2] + red[3];
  const float inv = 1.0f / sqrtf(ss / (float)H + eps);
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    const int n = (int)threadIdx.x * 4 + i * 1024;
    if (n >= H) continue;
    float out[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) out[c] = Act<T>::rnd(gv[i][c] * Act<T>::rnd(v[i][c] * inv));
    store4(hn + (size_t)row * H + n, out);
  }
}

template <typename T>
hipError_t launch_merge_norm_parts(const float* part, int kparts, int rows, int H, const float* x, const T* hsb,
                                   const T* hss, const T* rb, const T* rs, float* h, T* a_tap, const T* g2, T* hn,
                                   float eps, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (H > 4096 || H % 4) return hipErrorInvalidValue;
  switch ((H + 1023) / 1024) {
#define ZAYA_MNP_CASE(n)                                                                                          \
  case n:                                                                                                         \
    hipLaunchKernelGGL((merge_norm_parts_kernel<T, n>), dim3(rows), dim3(256), 0, s, part, kparts, rows, H, x, hsb, \
                       hss, rb, rs, h, a_tap, g2, hn, eps);                                                       \
    break;
    ZAYA_MNP_CASE(1) ZAYA_MNP_CASE(2) ZAYA_MNP_CASE(3) ZAYA_MNP_CASE(4)
#undef ZAYA_MNP_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_embed(const int32_t* ids, const T* table, const T* shift, const T* scale, float* x0, T* tap,
                        int rows, int H, int vocab, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(embed_kernel<T>, dim3((rows + 3) / 4), dim3(256), 0, s, ids, table, shift, scale, x0, tap, rows,
                     H, vocab);
  return hipGetLastError();
}

__global__ void fill_i32_kernel(int32_t* p, int n, int v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill_i32(int32_t* p, int n, int v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

template hipError_t launch_merge_norm_parts<bf16_t>(const float*, int, int, int, const float*, const bf16_t*,
                                                    const bf16_t*, const bf16_t*, const bf16_t*, float*, bf16_t*,
                                                    const bf16_t*, bf16_t*, float, hipStream_t);
template hipError_t launch_merge_norm_parts<float>(const float*, int, int, int, const float*, const float*, const float*,
                                                   const float*, const float*, float*, float*, const float*, float*,
                                                   float, hipStream_t);
template hipError_t launch_rmsnorm_stream<bf16_t>(const float*, const bf16_t*, bf16_t*, int, int, float, hipStream_t);
template hipError_t launch_rmsnorm_stream<float>(const float*, const float*, float*, int, int, float, hipStream_t);
template hipError_t launch_embed<bf16_t>(const int32_t*, const bf16_t*, const bf16_t*, const bf16_t*, float*, bf16_t*,
                                         int, int, int, hipStream_t);
template hipError_t launch_embed<float>(const int32_t*, const float*, const float*, const float*, float*, float*, int,
                                        int, int, hipStream_t);

}  // namespace zaya
