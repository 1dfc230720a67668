// Two-threshold block selection ("Block-Sparse Global Attention for Efficient
// Multi-View Geometry Transformers", key design 2; per-head budgets as in
// "HeSS: Head Sensitivity Score for Sparsity Redistribution in VGGT",
// proposed method).
//
// Per row of B probabilities: rank blocks by (probability desc, index asc),
// keep the first max(k_h, n_tau) where n_tau is the first n whose float64
// cumulative probability of the n top-ranked blocks reaches tau.
//
// Ranking key: (float32 bits of p) << 32 | (0xffffffff - j).  For p >= 0 the
// float bits order like the values, so the unique 64-bit keys sort in exactly
// the ranking order, and block j is kept iff key_j >= key of the last kept
// rank.  That threshold is all the compaction pass needs.
//
// Exactness of the cumulative sums: every float32 p >= 2^-29 is a multiple of
// 2^-52, so as long as the running sums stay below 2 every partial sum of
// such values is exact in float64, whatever the association.  The prefix up
// to the tau-crossing consists of values >= the crossing value, so the
// parallel scan here and a sequential sum reach identical decisions unless
// the crossing value itself is below 2^-29 (tau within ~B*2^-29 of the row's
// total).
#include <mutex>

#include "bsga_internal.hpp"

namespace bsga {

constexpr int kSelThreads = 256;

__device__ inline uint64_t rank_key(float p, int j) {
  return ((uint64_t)__float_as_uint(p) << 32) | (uint64_t)(0xffffffffu - (uint32_t)j);
}

__global__ __launch_bounds__(kSelThreads) void select_rows_kernel(
    const float* __restrict__ probs, int B, int n_pad, SelectParams sp,
    int32_t* __restrict__ counts, uint64_t* __restrict__ thresh) {
  extern __shared__ uint64_t keys[];  // n_pad entries
  __shared__ double wave_tot[kSelThreads / 64];
  __shared__ int s_ntau;
  const int row = blockIdx.x;
  const int h = row / B;
  const int T = threadIdx.x;
  const float* p = probs + (size_t)row * B;
  for (int j = T; j < n_pad; j += kSelThreads)
    keys[j] = j < B ? rank_key(p[j], j) : 0ull;
  if (T == 0) s_ntau = B;
  __syncthreads();

  // bitonic sort, descending
  for (int k = 2; k <= n_pad; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int idx = T; idx < (n_pad >> 1); idx += kSelThreads) {
        const int lo = ((idx & ~(jj - 1)) << 1) | (idx & (jj - 1));
        const int hi = lo + jj;
        const uint64_t a = keys[lo], b = keys[hi];
        const bool up = (lo & k) != 0;
        if (up ? (a > b) : (a < b)) {
          keys[lo] = b;
          keys[hi] = a;
        }
      }
      __syncthreads();
    }
  }

  // n_tau: cumulative float64 sum in rank order.  Thread T owns ranks
  // [T*C, (T+1)*C); padding keys are 0, i.e. probability 0.
  const double tau = sp.tau;
  int n_tau;
  if (tau <= 0.0) {
    n_tau = 0;
  } else if (tau >= 1.0) {
    n_tau = B;
  } else {
    const int C = n_pad / kSelThreads;  // n_pad >= kSelThreads
    double local = 0.0;
    for (int c = 0; c < C; ++c) local += (double)__uint_as_float((uint32_t)(keys[T * C + c] >> 32));
    // inclusive wave scan of the thread totals
    const int lane = T & 63, w = T >> 6;
    double incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    if (lane == 63) wave_tot[w] = incl;
    double excl = __shfl_up(incl, 1);
    if (lane == 0) excl = 0.0;
    __syncthreads();
    double base = 0.0;
    for (int u = 0; u < w; ++u) base += wave_tot[u];
    base += excl;
    double c_n = base;
    for (int c = 0; c < C; ++c) {
      c_n += (double)__uint_as_float((uint32_t)(keys[T * C + c] >> 32));
      if (c_n >= tau) {
        atomicMin(&s_ntau, T * C + c + 1);
        break;
      }
    }
    __syncthreads();
    n_tau = min(s_ntau, B);
  }
  if (T == 0) {
    const int count = min(B, max(sp.k[h], n_tau));
    counts[row] = count;
    thresh[row] = count > 0 ? keys[count - 1] : ~0ull;
  }
}

// The same selection with one wave per row, for rows of at most 512 blocks
// (up to 65,536 patch tokens at b = 128): the row's keys, padded to 512 with
// zeros (below every real key), stay in registers.  Sorted position
// i = 8 * lane + r lives in register r of the lane, so the bitonic network's
// partners i ^ j are registers of the same lane for j < 8 and the same
// register of lane ^ (j / 8) for j >= 8 (a cross-lane exchange): no LDS and no
// barriers.  The float64 prefix sums use a wave scan; the exactness argument
// above makes the decision independent of that association.
constexpr int kWaveRowKeys = 8;
constexpr int kWaveRowMax = 64 * kWaveRowKeys;

__device__ inline uint64_t xor_lanes(uint64_t x, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)x, m);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(x >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}

__global__ __launch_bounds__(256) void select_rows_wave_kernel(
    const float* __restrict__ probs, int B, int rows, SelectParams sp,
    int32_t* __restrict__ counts, uint64_t* __restrict__ thresh) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;  // uniform per wave
  const int h = row / B;
  const float* p = probs + (size_t)row * B;
  uint64_t key[kWaveRowKeys];
#pragma unroll
  for (int r = 0; r < kWaveRowKeys; ++r) {
    const int j = kWaveRowKeys * lane + r;
    key[r] = j < B ? rank_key(p[j], j) : 0ull;
  }
  // bitonic sort, descending: position i keeps the larger of the pair
  // (i, i ^ j) iff (i & j) == 0 equals (i & k) == 0
#pragma unroll
  for (int k = 2; k <= kWaveRowMax; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j < kWaveRowKeys) {
#pragma unroll
        for (int r = 0; r < kWaveRowKeys; ++r) {
          if (r & j) continue;
          const int i = kWaveRowKeys * lane + r;
          const bool desc = (i & k) == 0;
          const uint64_t a = key[r], b = key[r | j];
          const bool a_big = a > b;
          key[r] = (a_big == desc) ? a : b;
          key[r | j] = (a_big == desc) ? b : a;
        }
      } else {
        const int m = j / kWaveRowKeys;
        const bool lo = (lane & m) == 0;
        const bool desc = ((kWaveRowKeys * lane) & k) == 0;
#pragma unroll
        for (int r = 0; r < kWaveRowKeys; ++r) {
          const uint64_t other = xor_lanes(key[r], m);
          const bool keep_max = lo == desc;
          const bool mine_big = key[r] > other;
          key[r] = (mine_big == keep_max) ? key[r] : other;
        }
      }
    }
  }

  const double tau = sp.tau;
  int n_tau;
  if (tau <= 0.0) {
    n_tau = 0;
  } else if (tau >= 1.0) {
    n_tau = B;
  } else {
    double v[kWaveRowKeys], local = 0.0;
#pragma unroll
    for (int r = 0; r < kWaveRowKeys; ++r) {
      v[r] = (double)__uint_as_float((uint32_t)(key[r] >> 32));
      local += v[r];
    }
    double incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    double c_n = incl - local;  // exact: every partial sum here is exact
    int found = kWaveRowMax + 1;
#pragma unroll
    for (int r = 0; r < kWaveRowKeys; ++r) {
      c_n += v[r];
      if (found > kWaveRowMax && c_n >= tau) found = kWaveRowKeys * lane + r + 1;
    }
    // the running sums grow with the position, so the first lane that
    // reached tau holds the smallest such n
    const uint64_t hit = __ballot(found <= kWaveRowMax);
    n_tau = hit ? __shfl(found, __ffsll((unsigned long long)hit) - 1) : B;
    n_tau = min(n_tau, B);
  }
  const int count = min(B, max(sp.k[h], n_tau));
  uint64_t t = ~0ull;
  if (count > 0) {
    const int pos = count - 1, src = pos / kWaveRowKeys, reg = pos % kWaveRowKeys;
    uint64_t mine = key[0];
#pragma unroll
    for (int r = 1; r < kWaveRowKeys; ++r)
      if (reg == r) mine = key[r];
    const uint32_t lo32 = (uint32_t)__shfl((int)(uint32_t)mine, src);
    const uint32_t hi32 = (uint32_t)__shfl((int)(uint32_t)(mine >> 32), src);
    t = ((uint64_t)hi32 << 32) | lo32;
  }
  if (lane == 0) {
    counts[row] = count;
    thresh[row] = t;
  }
}

// Exclusive scan of the per-row counts into row_ptr (one workgroup).
__global__ __launch_bounds__(1024) void scan_counts_kernel(const int32_t* __restrict__ counts,
                                                           int rows,
                                                           int32_t* __restrict__ row_ptr) {
  __shared__ int wave_tot[16];
  const int T = threadIdx.x;
  const int per = (rows + 1023) / 1024;
  const int lo = min(rows, T * per), hi = min(rows, lo + per);
  int local = 0;
  for (int r = lo; r < hi; ++r) local += counts[r];
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
  for (int r = lo; r < hi; ++r) {
    row_ptr[r] = run;
    run += counts[r];
  }
  if (T == 1023) row_ptr[rows] = run;
}

// Ascending compaction: block j of row r is kept iff its key >= thresh[r].
__global__ __launch_bounds__(256) void expand_kernel(const float* __restrict__ probs, int B,
                                                     int rows,
                                                     const uint64_t* __restrict__ thresh,
                                                     const int32_t* __restrict__ row_ptr,
                                                     int32_t* __restrict__ col_idx) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float* p = probs + (size_t)row * B;
  const uint64_t thr = thresh[row];
  int out = row_ptr[row];
  for (int j0 = 0; j0 < B; j0 += 64) {
    const int j = j0 + lane;
    const bool keep = j < B && rank_key(p[j], j) >= thr;
    const uint64_t mask = __ballot(keep);
    if (keep) {
      const int pos = __popcll(mask & ((1ull << lane) - 1ull));
      col_idx[out + pos] = j;
    }
    out += __popcll(mask);
  }
}

static int pow2_at_least(int x) {
  int n = kSelThreads;
  while (n < x) n <<= 1;
  return n;
}

size_t select_workspace(const Dims& d) {
  const size_t rows = (size_t)d.H * d.B;
  size_t a = ((rows * sizeof(int32_t)) + 255) & ~(size_t)255;
  return a + rows * sizeof(uint64_t);
}

hipError_t launch_select(const Dims& d, const float* probs, const SelectParams& sp,
                         int32_t* row_ptr, int32_t* col_idx, void* ws, hipStream_t st) {
  const int rows = d.H * d.B;
  int32_t* counts = (int32_t*)ws;
  uint64_t* thresh =
      (uint64_t*)((char*)ws + ((((size_t)rows * sizeof(int32_t)) + 255) & ~(size_t)255));
  if (d.B <= kWaveRowMax) {
    select_rows_wave_kernel<<<(rows + 3) / 4, 256, 0, st>>>(probs, d.B, rows, sp, counts,
                                                             thresh);
  } else {
    const int n_pad = pow2_at_least(d.B);
    select_rows_kernel<<<rows, kSelThreads, n_pad * sizeof(uint64_t), st>>>(
        probs, d.B, n_pad, sp, counts, thresh);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  scan_counts_kernel<<<1, 1024, 0, st>>>(counts, rows, row_ptr);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  expand_kernel<<<(rows + 3) / 4, 256, 0, st>>>(probs, d.B, rows, thresh, row_ptr, col_idx);
  return hipGetLastError();
}

hipError_t launch_scan_counts(const int32_t* counts, int rows, int32_t* row_ptr, hipStream_t st) {
  scan_counts_kernel<<<1, 1024, 0, st>>>(counts, rows, row_ptr);
  return hipGetLastError();
}

}  // namespace bsga

namespace bsga {

// ---------------------------------------------------------------------------
// Selection without a caller workspace (bsga_select_static).  The per-row
// counts and thresholds live in `scratch`, a file-scope device array: one
// copy per GPU, held until the process ends, shared by every such call on
// that GPU (calls that overlap on one GPU race on it).  Each row kernel
// writes its row's count and threshold before the scan and the compaction
// read them, so nothing in it has to start at zero and leftovers of an
// earlier call are never read.
constexpr size_t kStaticScratchBytes = size_t(1) << 20;
static_assert((((size_t)BSGA_SELECT_STATIC_MAX_ROWS * sizeof(int32_t) + 255) & ~(size_t)255) +
                      (size_t)BSGA_SELECT_STATIC_MAX_ROWS * sizeof(uint64_t) <=
                  kStaticScratchBytes,
              "scratch holds the largest accepted selection");
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
hipError_t select_static_scratch(void** out, size_t* bytes) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  *bytes = kStaticScratchBytes;
  return hipSuccess;
}

}  // namespace bsga
