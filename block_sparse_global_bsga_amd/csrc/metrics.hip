// Normalised mean squared error of an attention output against a reference
// ("SAF3R: Dynamic Sparse Attention for Feed-Forward 3D Reconstruction
// Transformers", section 4, offline head profiling: the error of a sparse
// configuration is ||O_full - O_sparse||^2 / ||O_full||^2 per head).
//
// Memory-bound: both [H][N][64] bf16 tensors are read once.  Each workgroup
// reduces one chunk of a head in float32 (16-byte loads, eight values per
// lane per step) into a float64 pair; a second kernel adds the chunks of each
// head in chunk order (deterministic) and divides.
#include "bsga_internal.hpp"

namespace bsga {

constexpr int kNmseVecs = 8192;  // 16-byte vectors per chunk (= 1024 token rows)

__global__ __launch_bounds__(256) void nmse_partial_kernel(const uint4* __restrict__ ref,
                                                           const uint4* __restrict__ out,
                                                           double* __restrict__ partial,
                                                           size_t vecs_per_head, int chunks) {
  __shared__ double red[2][4];
  const int c = blockIdx.x, h = blockIdx.y, T = threadIdx.x;
  const size_t base = (size_t)h * vecs_per_head;
  const size_t lo = (size_t)c * kNmseVecs;
  const size_t hi = lo + kNmseVecs < vecs_per_head ? lo + kNmseVecs : vecs_per_head;
  float num = 0.f, den = 0.f;
  for (size_t i = lo + T; i < hi; i += 256) {
    const uint4 a = ref[base + i], b = out[base + i];
    const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float r0 = __uint_as_float(wa[e] << 16), r1 = __uint_as_float(wa[e] & 0xffff0000u);
      const float o0 = __uint_as_float(wb[e] << 16), o1 = __uint_as_float(wb[e] & 0xffff0000u);
      num = fmaf(r0 - o0, r0 - o0, num);
      num = fmaf(r1 - o1, r1 - o1, num);
      den = fmaf(r0, r0, den);
      den = fmaf(r1, r1, den);
    }
  }
  double dn = num, dd = den;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    dn += __shfl_xor(dn, off);
    dd += __shfl_xor(dd, off);
  }
  if ((T & 63) == 0) {
    red[0][T >> 6] = dn;
    red[1][T >> 6] = dd;
  }
  __syncthreads();
  if (T == 0) {
    partial[((size_t)h * chunks + c) * 2] = red[0][0] + red[0][1] + red[0][2] + red[0][3];
    partial[((size_t)h * chunks + c) * 2 + 1] = red[1][0] + red[1][1] + red[1][2] + red[1][3];
  }
}

__global__ __launch_bounds__(64) void nmse_final_kernel(const double* __restrict__ partial,
                                                        int heads, int chunks,
                                                        double* __restrict__ result) {
  const int h = blockIdx.x * 64 + threadIdx.x;
  if (h >= heads) return;
  double num = 0.0, den = 0.0;
  for (int c = 0; c < chunks; ++c) {
    num += partial[((size_t)h * chunks + c) * 2];
    den += partial[((size_t)h * chunks + c) * 2 + 1];
  }
  result[h] = den > 0.0 ? num / den : (num > 0.0 ? INFINITY : 0.0);
}

int nmse_chunks(const Dims& d) {
  const size_t vecs = (size_t)d.n * 8;
  return (int)((vecs + kNmseVecs - 1) / kNmseVecs);
}

size_t nmse_workspace(const Dims& d) { return (size_t)d.H * nmse_chunks(d) * 2 * sizeof(double); }

hipError_t launch_nmse(const Dims& d, const uint16_t* ref, const uint16_t* out, double* result,
                       void* ws, hipStream_t st) {
  const int chunks = nmse_chunks(d);
  double* partial = (double*)ws;
  nmse_partial_kernel<<<dim3(chunks, d.H), 256, 0, st>>>((const uint4*)ref, (const uint4*)out,
                                                         partial, (size_t)d.n * 8, chunks);
  nmse_final_kernel<<<(d.H + 63) / 64, 64, 0, st>>>(partial, d.H, chunks, result);
  return hipGetLastError();
}

}  // namespace bsga
