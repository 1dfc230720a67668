// Block-mask prediction: block average pooling of Q and K, the pooled score
// product S = Qbar Kbar^T / sqrt(64), and a row softmax over key blocks.
// Follows "Block-Sparse Global Attention for Efficient Multi-View Geometry
// Transformers", key design 1 (a low-resolution attention map from pooled Q
// and K; no learned parameters).
#include "bsga_internal.hpp"

namespace bsga {

// ---------------------------------------------------------------------------
// Pooling.  One workgroup per (query block i, head h) reads the block's patch
// rows of Q and K with 16-byte loads (8 lanes per 128-byte row, 32 rows per
// pass) and writes both float32 means.  Memory-bound: every byte is read once.
template <int BLK>
__global__ __launch_bounds__(256) void pool_kernel(const uint4* __restrict__ q,
                                                   const uint4* __restrict__ k,
                                                   float* __restrict__ qbar,
                                                   float* __restrict__ kbar,
                                                   Dims d) {
  constexpr int kPass = BLK / 32;
  const int i = blockIdx.x, h = blockIdx.y, T = threadIdx.x;
  const int chunk = T & 7, row0 = T >> 3;
  const int p0 = i * BLK;
  const int nvalid = min(BLK, d.np - p0);
  const size_t head = (size_t)h * d.n * 8;  // uint4 units, 8 per token row

  uint4 vq[kPass], vk[kPass];
#pragma unroll
  for (int r = 0; r < kPass; ++r) {
    const int row = row0 + 32 * r;
    if (row < nvalid) {
      const size_t t = patch_token(p0 + row, d);
      vq[r] = q[head + t * 8 + chunk];
      vk[r] = k[head + t * 8 + chunk];
    } else {
      vq[r] = make_uint4(0, 0, 0, 0);
      vk[r] = make_uint4(0, 0, 0, 0);
    }
  }
  float aq[8], ak[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) aq[e] = ak[e] = 0.f;
#pragma unroll
  for (int r = 0; r < kPass; ++r) {
    const uint32_t wq[4] = {vq[r].x, vq[r].y, vq[r].z, vq[r].w};
    const uint32_t wk[4] = {vk[r].x, vk[r].y, vk[r].z, vk[r].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      aq[2 * e] += __uint_as_float(wq[e] << 16);
      aq[2 * e + 1] += __uint_as_float(wq[e] & 0xffff0000u);
      ak[2 * e] += __uint_as_float(wk[e] << 16);
      ak[2 * e + 1] += __uint_as_float(wk[e] & 0xffff0000u);
    }
  }
  // Reduce the 8 row groups of a wave (lanes sharing `chunk`), then the waves.
#pragma unroll
  for (int off = 8; off < 64; off <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      aq[e] += __shfl_xor(aq[e], off);
      ak[e] += __shfl_xor(ak[e], off);
    }
  }
  __shared__ float red[2][4][64];
  const int w = T >> 6, lane = T & 63;
  if (lane < 8) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      red[0][w][lane * 8 + e] = aq[e];
      red[1][w][lane * 8 + e] = ak[e];
    }
  }
  __syncthreads();
  if (T < 128) {
    const int which = T >> 6, c = T & 63;
    const float s = ((red[which][0][c] + red[which][1][c]) + red[which][2][c]) +
                    red[which][3][c];
    float* out = which ? kbar : qbar;
    out[((size_t)h * d.B + i) * kHeadDim + c] = s / (float)nvalid;
  }
}

hipError_t launch_pool(const Dims& d, const uint16_t* q, const uint16_t* k,
                       float* qbar, float* kbar, hipStream_t st) {
  dim3 grid(d.B, d.H);
  if (d.b == 64)
    pool_kernel<64><<<grid, 256, 0, st>>>((const uint4*)q, (const uint4*)k,
                                          qbar, kbar, d);
  else
    pool_kernel<128><<<grid, 256, 0, st>>>((const uint4*)q, (const uint4*)k,
                                           qbar, kbar, d);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Pooled scores on bf16 MFMA.  Each float32 mean is split exactly-enough into
// three bf16 terms x = x1 + x2 + x3 (each the rounded remainder of the last);
// the six products x_a y_b with a + b <= 4 are accumulated in float32, which
// leaves an error near float32 rounding of the dot product.
//
// Operand layout of v_mfma_f32_32x32x16_bf16: lane l supplies A row (l % 32)
// and B column (l % 32), eight k-values each, the two half-waves covering two
// disjoint k-groups.  The head dimension is the contraction, so any fixed
// assignment of dimensions to k-slots works; half-wave hh takes dimensions
// [32 hh, 32 hh + 32), eight per instruction.
__device__ inline void split3(const float* x, bf16x8& a, bf16x8& b, bf16x8& c) {
  f32x8 v, r1, r2;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = x[e];
  a = __builtin_convertvector(v, bf16x8);
  r1 = v - __builtin_convertvector(a, f32x8);
  b = __builtin_convertvector(r1, bf16x8);
  r2 = r1 - __builtin_convertvector(b, f32x8);
  c = __builtin_convertvector(r2, bf16x8);
}

// s receives S (the softmax then runs on it in place); s2, when not null, a
// copy of S for the caller.
__global__ __launch_bounds__(256) void scores_kernel(const float* __restrict__ qbar,
                                                     const float* __restrict__ kbar,
                                                     float* __restrict__ s, float* __restrict__ s2,
                                                     Dims d) {
  const int h = blockIdx.z;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const int i0 = blockIdx.y * 64 + 32 * (w >> 1);
  const int j0 = blockIdx.x * 64 + 32 * (w & 1);
  const float* qrow = qbar + ((size_t)h * d.B + min(i0 + l32, d.B - 1)) * kHeadDim + 32 * hh;
  const float* krow = kbar + ((size_t)h * d.B + min(j0 + l32, d.B - 1)) * kHeadDim + 32 * hh;
  f32x16 acc = {};
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    float xq[8], xk[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      xq[e] = qrow[8 * m + e];
      xk[e] = krow[8 * m + e];
    }
    bf16x8 q1, q2, q3, k1, k2, k3;
    split3(xq, q1, q2, q3);
    split3(xk, k1, k2, k3);
    // small terms first
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q1, k3, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q3, k1, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q2, k2, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q1, k2, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q2, k1, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q1, k1, acc, 0, 0, 0);
  }
  // acc[r] holds S[i0 + 8(r/4) + 4 hh + r%4][j0 + l32]
  const int j = j0 + l32;
  if (j < d.B) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = i0 + 8 * (r >> 2) + 4 * hh + (r & 3);
      if (i < d.B) {
        const size_t at = ((size_t)h * d.B + i) * d.B + j;
        s[at] = acc[r] * 0.125f;
        if (s2) s2[at] = acc[r] * 0.125f;
      }
    }
  }
}

hipError_t launch_scores(const Dims& d, const float* qbar, const float* kbar,
                         float* probs, float* scores, hipStream_t st) {
  const int t = (d.B + 63) / 64;
  scores_kernel<<<dim3(t, t, d.H), 256, 0, st>>>(qbar, kbar, probs, scores, d);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Row softmax in place, one wave per row of B scores (max-subtracted, float32,
// IEEE exp and division; fixed reduction order, so results are reproducible).
__device__ inline float wave_max(float x) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}
__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off);
  return x;
}

__global__ __launch_bounds__(256) void softmax_kernel(float* __restrict__ p,
                                                      int rows, int B) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  float* r = p + (size_t)row * B;
  float m = -INFINITY;
  for (int j = lane; j < B; j += 64) m = fmaxf(m, r[j]);
  m = wave_max(m);
  float s = 0.f;
  for (int j = lane; j < B; j += 64) {
    const float e = expf(r[j] - m);
    r[j] = e;
    s += e;
  }
  s = wave_sum(s);
  for (int j = lane; j < B; j += 64) r[j] = r[j] / s;
}

hipError_t launch_softmax(const Dims& d, float* probs, hipStream_t st) {
  const int rows = d.H * d.B;
  softmax_kernel<<<(rows + 3) / 4, 256, 0, st>>>(probs, rows, d.B);
  return hipGetLastError();
}

}  // namespace bsga
