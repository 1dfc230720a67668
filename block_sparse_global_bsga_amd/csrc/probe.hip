// Query-probe Top-K block selection ("SAF3R: Dynamic Sparse Attention for
// Feed-Forward 3D Reconstruction Transformers", section 4: query-probe Top-K
// kernel and its online estimate).  The mean over queries of a key's score
// q_i . k_t / sqrt(d) is the score of that key against the mean query, so one
// probe vector qbar = (1/N) sum_i q_i ranks every key in O(N).  Here the
// ranked keys are the patch keys, the top `topk` of them (score descending,
// lower patch index first) are kept, and every query block of the head keeps
// the patch blocks that hold at least one of them (block lists for the
// block-sparse attention kernel; the special keys stay dense as always).
//
//   probe_partial_kernel : per (head, chunk of 256 tokens) float32 column sums
//                          of Q (HBM-bound: reads Q once)
//   probe_mean_kernel    : per head, the chunk sums in chunk order / N -> qbar
//   probe_scores_kernel  : per patch key, qbar . k / 8 (HBM-bound: reads the
//                          patch rows of K once)
//   probe_topk_kernel    : per head, exact radix select of the topk-th largest
//                          64-bit key (score bits, inverted index), then the
//                          ascending list of blocks holding a key >= it
//   probe_emit_kernel    : CSR rows (every row of a head gets that list)
#include "bsga_internal.hpp"

namespace bsga {

constexpr int kProbeRows = 256;  // tokens per partial-sum chunk

// 8 lanes per 128-byte row, 32 rows per pass of a 256-thread workgroup.
__global__ __launch_bounds__(256) void probe_partial_kernel(const uint4* __restrict__ q,
                                                            float* __restrict__ partial,
                                                            Dims d, int chunks) {
  __shared__ float red[32][65];
  const int c = blockIdx.x, h = blockIdx.y, T = threadIdx.x;
  const int ch = T & 7, r0 = T >> 3;
  const size_t head = (size_t)h * d.n * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int t_end = min(d.n, (c + 1) * kProbeRows);
  for (int t = c * kProbeRows + r0; t < t_end; t += 32) {
    const uint4 v = q[head + (size_t)t * 8 + ch];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += __uint_as_float(w[e] << 16);
      acc[2 * e + 1] += __uint_as_float(w[e] & 0xffff0000u);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[r0][ch * 8 + e] = acc[e];
  __syncthreads();
  if (T < 64) {
    float s = 0.f;
    for (int r = 0; r < 32; ++r) s += red[r][T];
    partial[((size_t)h * chunks + c) * kHeadDim + T] = s;
  }
}

__global__ __launch_bounds__(64) void probe_mean_kernel(const float* __restrict__ partial,
                                                        float* __restrict__ qbar, Dims d,
                                                        int chunks) {
  const int h = blockIdx.x, T = threadIdx.x;
  float s = 0.f;
  for (int c = 0; c < chunks; ++c) s += partial[((size_t)h * chunks + c) * kHeadDim + T];
  qbar[h * kHeadDim + T] = s / (float)d.n;
}

// One 8-lane group per patch key: 16-byte slice dot products reduced by
// xor shuffles.  Scores are written in patch order.
__global__ __launch_bounds__(256) void probe_scores_kernel(const uint4* __restrict__ k,
                                                           const float* __restrict__ qbar,
                                                           float* __restrict__ scores, Dims d) {
  const int h = blockIdx.y, T = threadIdx.x;
  const int ch = T & 7;
  float qv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) qv[e] = qbar[h * kHeadDim + ch * 8 + e];
  const size_t head = (size_t)h * d.n * 8;
  for (int p = blockIdx.x * 32 + (T >> 3); p < d.np; p += gridDim.x * 32) {
    const uint32_t t = patch_token((uint32_t)p, d);
    const uint4 v = k[head + (size_t)t * 8 + ch];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s = fmaf(__uint_as_float(w[e] << 16), qv[2 * e], s);
      s = fmaf(__uint_as_float(w[e] & 0xffff0000u), qv[2 * e + 1], s);
    }
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 4);
    if (ch == 0) scores[(size_t)h * d.np + p] = s * 0.125f;
  }
}

// Order-preserving 64-bit key: float bits made monotone (-0 folded into +0),
// then the inverted patch index so that lower indices rank higher.
__device__ inline uint64_t probe_key(float s, int p) {
  if (s == 0.f) s = 0.f;
  const uint32_t b = __float_as_uint(s);
  const uint32_t m = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)m << 32) | (uint64_t)(0xffffffffu - (uint32_t)p);
}

constexpr int kTopkThreads = 1024;

__global__ __launch_bounds__(kTopkThreads) void probe_topk_kernel(const float* __restrict__ scores,
                                                                  Dims d, int topk,
                                                                  int32_t* __restrict__ list,
                                                                  int32_t* __restrict__ count) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t bin_tot[4];
  __shared__ uint64_t s_prefix;
  __shared__ int s_rem, s_done;
  __shared__ uint8_t keep[BSGA_MAX_BLOCKS];
  __shared__ int wave_tot[kTopkThreads / 64];
  const int h = blockIdx.x, T = threadIdx.x;
  const float* sc = scores + (size_t)h * d.np;
  const int K = min(topk, d.np);
  for (int j = T; j < d.B; j += kTopkThreads) keep[j] = 0;
  if (T == 0) {
    s_prefix = 0;
    s_rem = K;
    s_done = 0;
  }
  __syncthreads();
  if (K > 0) {
    // MSB-first radix select, 8 bits per pass: after pass d the top 8(d+1)
    // bits of the K-th largest key are known.  When the K-th largest falls in
    // a bin that must be taken whole (every key with that prefix is among the
    // top K), the prefix itself is the threshold and the select stops early;
    // without ties in the scores that happens after the 4 score-bit passes.
    for (int pass = 0; pass < 8; ++pass) {
      const int shift = 56 - 8 * pass;
      const uint64_t hi_mask = pass == 0 ? 0ull : (~0ull << (shift + 8));
      const uint64_t prefix = s_prefix;
      for (int i = T; i < 256; i += kTopkThreads) hist[i] = 0;
      __syncthreads();
      for (int p = T; p < d.np; p += kTopkThreads) {
        const uint64_t key = probe_key(sc[p], p);
        if ((key & hi_mask) == prefix) atomicAdd(&hist[(key >> shift) & 255], 1u);
      }
      __syncthreads();
      // thread T < 256 takes bin 255 - T: an inclusive scan over T counts the
      // keys in that bin and every higher one
      const int rem = s_rem;
      uint32_t own = 0, incl = 0;
      if (T < 256) {
        own = hist[255 - T];
        incl = own;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const uint32_t o = __shfl_up(incl, off);
          if ((T & 63) >= off) incl += o;
        }
        if ((T & 63) == 63) bin_tot[T >> 6] = incl;
      }
      __syncthreads();
      if (T < 256) {
        for (int u = 0; u < (T >> 6); ++u) incl += bin_tot[u];
        // the bin where the running count first reaches rem
        if (incl >= (uint32_t)rem && incl - own < (uint32_t)rem) {
          const uint32_t left = (uint32_t)rem - (incl - own);
          s_prefix = prefix | ((uint64_t)(255 - T) << shift);
          s_rem = (int)left;
          s_done = left == own;
        }
      }
      __syncthreads();
      if (s_done) break;
    }
    const uint64_t thr = s_prefix;  // the K-th largest key
    for (int p = T; p < d.np; p += kTopkThreads)
      if (probe_key(sc[p], p) >= thr) keep[p / d.b] = 1;
  }
  __syncthreads();
  // ascending compaction of the kept blocks
  const int per = (d.B + kTopkThreads - 1) / kTopkThreads;
  const int lo = min(d.B, T * per), hi = min(d.B, lo + per);
  int local = 0;
  for (int j = lo; j < hi; ++j) local += keep[j];
  const int lane = T & 63, w = T >> 6;
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wave_tot[w] = incl;
  __syncthreads();
  int run = incl - local;
  for (int u = 0; u < w; ++u) run += wave_tot[u];
  for (int j = lo; j < hi; ++j)
    if (keep[j]) list[(size_t)h * d.B + run++] = j;
  if (T == kTopkThreads - 1) count[h] = run;
}

// Row (h, i): row_ptr = sum over earlier heads of B * count + i * count[h];
// the columns are the head's list.
__global__ __launch_bounds__(256) void probe_emit_kernel(const int32_t* __restrict__ list,
                                                         const int32_t* __restrict__ count,
                                                         Dims d, int32_t* __restrict__ row_ptr,
                                                         int32_t* __restrict__ col_idx) {
  const int i = blockIdx.x, h = blockIdx.y, T = threadIdx.x;
  int64_t base = 0;
  for (int u = 0; u < h; ++u) base += (int64_t)d.B * count[u];
  const int n = count[h];
  const int64_t off = base + (int64_t)i * n;
  if (T == 0) row_ptr[h * d.B + i] = (int32_t)off;
  if (T == 0 && h == d.H - 1 && i == d.B - 1) row_ptr[d.H * d.B] = (int32_t)(off + n);
  for (int j = T; j < n; j += 256) col_idx[off + j] = list[(size_t)h * d.B + j];
}

int probe_chunks(const Dims& d) { return (d.n + kProbeRows - 1) / kProbeRows; }

size_t probe_workspace(const Dims& d) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return up((size_t)d.H * probe_chunks(d) * kHeadDim * sizeof(float)) +   // partial sums
         up((size_t)d.H * kHeadDim * sizeof(float)) +                       // qbar
         up((size_t)d.H * d.np * sizeof(float)) +                           // scores
         up((size_t)d.H * d.B * sizeof(int32_t)) +                          // block lists
         up((size_t)d.H * sizeof(int32_t));                                 // counts
}

hipError_t launch_probe_select(const Dims& d, const uint16_t* q, const uint16_t* k, int topk,
                               float* scores_out, int32_t* row_ptr, int32_t* col_idx, void* ws,
                               hipStream_t st) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const int chunks = probe_chunks(d);
  char* p = (char*)ws;
  float* partial = (float*)p;
  p += up((size_t)d.H * chunks * kHeadDim * sizeof(float));
  float* qbar = (float*)p;
  p += up((size_t)d.H * kHeadDim * sizeof(float));
  float* scores = (float*)p;
  p += up((size_t)d.H * d.np * sizeof(float));
  int32_t* list = (int32_t*)p;
  p += up((size_t)d.H * d.B * sizeof(int32_t));
  int32_t* count = (int32_t*)p;
  if (scores_out) scores = scores_out;

  probe_partial_kernel<<<dim3(chunks, d.H), 256, 0, st>>>((const uint4*)q, partial, d, chunks);
  probe_mean_kernel<<<d.H, 64, 0, st>>>(partial, qbar, d, chunks);
  const int sblocks = min((d.np + 31) / 32, 2048);
  probe_scores_kernel<<<dim3(sblocks, d.H), 256, 0, st>>>((const uint4*)k, qbar, scores, d);
  probe_topk_kernel<<<d.H, kTopkThreads, 0, st>>>(scores, d, topk, list, count);
  probe_emit_kernel<<<dim3(d.B, d.H), 256, 0, st>>>(list, count, d, row_ptr, col_idx);
  return hipGetLastError();
}

}  // namespace bsga
