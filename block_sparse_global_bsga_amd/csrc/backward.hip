// Backward of the layer's attention for a fixed block mask (the outlook of
// "Block-Sparse Global Attention for Efficient Multi-View Geometry
// Transformers": sparse attention inside training).  The mask is the one the
// forward used: patch queries see the patch tokens of their kept blocks and
// every special token; special queries see every token.  The block selection
// is not differentiated.
//
// With the forward's LSE, per allowed (query, key): P = exp(q.k/8 - LSE),
// dP = dO . v, D = dO . O (per query), dS = P (dP - D), and
//   dQ = sum_k dS k / 8,  dK = sum_q dS q / 8,  dV = sum_q P dO.
//
// Layout: every operand is first packed (the forward's packed order: patch
// tokens, pad, special tokens, pad) both as rows [H][Ntot][64] and, where a
// product contracts over tokens, transposed [H][64][Ntot], so that tiles
// stream into LDS with direct-to-LDS loads exactly as in the forward.
//
// dq_kernel (query-major, over the CSR rows): per wave 32 queries with Q and
//   dO rows in registers; per key tile S^T = K Q^T and dP^T = V dO^T (K, V
//   rows from LDS), dS^T in the accumulator layout, dQ^T += K^T dS^T with dS^T
//   taken straight from the accumulators as the B operand (K row permutation
//   pi, as in the forward).
// dkdv_kernel (key-major, over the transposed CSR): per wave 32 keys with K
//   and V rows in registers; per query tile S = Q K^T and dP = dO V^T (Q, dO
//   rows from LDS, row permutation pi), then dV^T += dO^T P and
//   dK^T += Q^T dS from the accumulators.  There P carries a factor 2^15
//   (exp2 against LSE - 15) so that every weight that matters is a normal
//   float16 number, and dV^T += dO^T P runs on float16 MFMA with dO^T stored
//   as float16 times a per-head power of two 2^sigma (its largest |dO| in
//   [2^14, 2^15)): P enters once, rounded to 11 significant bits, while dS
//   still enters dK as a bf16 pair hi + lo.  The epilogue undoes 2^15 (dK)
//   and 2^(15 + sigma) (dV).
#include <type_traits>

#include "bsga_internal.hpp"
#include "tile_common.hpp"

namespace bsga {

typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) void lds_void;

// dkdv_kernel's weights are 2^kPScaleLog2 P: every weight above 2^-29 is a
// normal float16 number, and none exceeds 2^15
constexpr float kPScaleLog2 = 15.f;

// ---------------------------------------------------------------------------
// Packing: rows and/or transposed copies of one [H][N][64] tensor in packed
// order, 64 tokens per workgroup (zeros for padding).
// With chunk_max given, the transposed copy holds float16 x * 2^sigma_h
// (sigma_h from the head's largest |x|, written to sig[h]) instead of bf16.
__global__ __launch_bounds__(256) void bwd_pack_kernel(const uint4* __restrict__ x,
                                                       uint4* __restrict__ rows,
                                                       uint4* __restrict__ cols, Dims d,
                                                       const uint32_t* __restrict__ chunk_max,
                                                       int* __restrict__ sig, int nchunk) {
  __shared__ uint16_t sv[64][66];
  __shared__ int sig_s;
  const int kp0 = wg_x() * 64, h = wg_y(), T = lid_x();
  if (chunk_max != nullptr && T < 64) {
    const int sg = head_sigma(chunk_max, h, nchunk, T);
    if (T == 0) {
      sig_s = sg;
      if (wg_x() == 0) sig[h] = sg;
    }
  }
  const size_t src_head = (size_t)h * d.n * 8;
  uint4 vv[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = T + 256 * i;
    const int row = c >> 3, ch = c & 7;
    const int tok = packed_token(kp0 + row, d);
    vv[i] = make_uint4(0, 0, 0, 0);
    if (tok >= 0) vv[i] = x[src_head + (size_t)tok * 8 + ch];
    if (rows) rows[((size_t)h * d.ntot_pad + kp0 + row) * 8 + ch] = vv[i];
  }
  if (!cols) return;
  __syncthreads();  // sig_s
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = T + 256 * i;
    const int row = c >> 3, ch = c & 7;
    const uint32_t w[4] = {vv[i].x, vv[i].y, vv[i].z, vv[i].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint16_t lo = (uint16_t)(w[e] & 0xffff), hi = (uint16_t)(w[e] >> 16);
      if (chunk_max != nullptr) {
        // bf16 -> float32 (exact) -> times 2^sigma (exact) -> float16 (exact in range)
        lo = __builtin_bit_cast(uint16_t,
                                (_Float16)__builtin_amdgcn_ldexpf(__uint_as_float(w[e] << 16), sig_s));
        hi = __builtin_bit_cast(uint16_t, (_Float16)__builtin_amdgcn_ldexpf(
                                              __uint_as_float(w[e] & 0xffff0000u), sig_s));
      }
      sv[row][ch * 8 + 2 * e] = lo;
      sv[row][ch * 8 + 2 * e + 1] = hi;
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = T + 256 * i;
    const int dr = c >> 3, kc = c & 7;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)sv[8 * kc + 2 * e][dr] | ((uint32_t)sv[8 * kc + 2 * e + 1][dr] << 16);
    cols[(((size_t)h * 64 + dr) * d.ntot_pad + kp0) / 8 + kc] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Per packed row: lse2 = LSE * log2(e) (+inf for padding, so every weight of
// a padding row is 0), lse2s = lse2 - 15 (the weights 2^15 P of dkdv_kernel)
// and D = dO . O in float32 (0 for padding), from the bf16 rows o or, when
// given, the float32 rows o32 of the training-mode forward.  Without o32,
// dq_kernel overwrites D for every row of its query tiles with sum_k P dP;
// rows no query tile covers are padding and keep 0.
__global__ __launch_bounds__(256) void bwd_rowstats_kernel(const uint4* __restrict__ o,
                                                           const float4* __restrict__ o32,
                                                           const uint4* __restrict__ d_o,
                                                           const float* __restrict__ lse,
                                                           float* __restrict__ lse2,
                                                           float* __restrict__ lse2s,
                                                           float* __restrict__ dd, Dims d) {
  const int h = wg_y(), T = lid_x(), ch = T & 7;
  const int kp = wg_x() * 32 + (T >> 3);  // 32 rows per workgroup, 8 lanes per row
  const int tok = packed_token(kp, d);
  float s = 0.f;
  if (tok >= 0) {
    const size_t at = ((size_t)h * d.n + tok) * 8 + ch;
    const uint4 b = d_o[at];
    const uint32_t wb[4] = {b.x, b.y, b.z, b.w};
    if (o32 != nullptr) {
      // dims 8 ch .. 8 ch + 7 of the row as two float4
      const float4 x0 = o32[at * 2], x1 = o32[at * 2 + 1];
      const float xo[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s = fmaf(xo[2 * e], __uint_as_float(wb[e] << 16), s);
        s = fmaf(xo[2 * e + 1], __uint_as_float(wb[e] & 0xffff0000u), s);
      }
    } else {
      const uint4 a = o[at];
      const uint32_t wa[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s = fmaf(__uint_as_float(wa[e] << 16), __uint_as_float(wb[e] << 16), s);
        s = fmaf(__uint_as_float(wa[e] & 0xffff0000u), __uint_as_float(wb[e] & 0xffff0000u), s);
      }
    }
  }
  s += __shfl_xor(s, 1);
  s += __shfl_xor(s, 2);
  s += __shfl_xor(s, 4);
  if (ch == 0) {
    const size_t r = (size_t)h * d.ntot_pad + kp;
    dd[r] = s;
    const float l2 = tok >= 0 ? lse[(size_t)h * d.n + tok] * 1.4426950408889634f : INFINITY;
    lse2[r] = l2;
    lse2s[r] = l2 - kPScaleLog2;
  }
}

// ---------------------------------------------------------------------------
// Transposed CSR: for key block j of head h, the query blocks i (ascending)
// whose kept list holds j.
__device__ inline bool row_has(const int32_t* __restrict__ cols, int n, int j) {
  int lo = 0, hi = n;  // sorted ascending
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (cols[mid] < j) lo = mid + 1; else hi = mid;
  }
  return lo < n && cols[lo] == j;
}

__global__ __launch_bounds__(256) void csr_t_count_kernel(const int32_t* __restrict__ row_ptr,
                                                          const int32_t* __restrict__ col_idx,
                                                          Dims d, int32_t* __restrict__ count) {
  __shared__ int red[4];
  const int j = wg_x(), h = wg_y(), T = lid_x();
  int c = 0;
  for (int i = T; i < d.B; i += 256) {
    const int r = h * d.B + i;
    const int a = row_ptr[r];
    c += row_has(col_idx + a, max(0, min(row_ptr[r + 1] - a, d.B)), j);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
  if ((T & 63) == 0) red[T >> 6] = c;
  __syncthreads();
  if (T == 0) count[h * d.B + j] = red[0] + red[1] + red[2] + red[3];
}

__global__ __launch_bounds__(256) void csr_t_fill_kernel(const int32_t* __restrict__ row_ptr,
                                                         const int32_t* __restrict__ col_idx,
                                                         const int32_t* __restrict__ t_ptr, Dims d,
                                                         int32_t* __restrict__ t_list) {
  __shared__ int wave_tot[4];
  const int j = wg_x(), h = wg_y(), T = lid_x();
  const int per = (d.B + 255) / 256;
  const int lo = min(d.B, T * per), hi = min(d.B, lo + per);
  int local = 0;
  for (int i = lo; i < hi; ++i) {
    const int r = h * d.B + i, a = row_ptr[r];
    local += row_has(col_idx + a, max(0, min(row_ptr[r + 1] - a, d.B)), j);
  }
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
  int32_t* out = t_list + t_ptr[h * d.B + j];
  for (int i = lo; i < hi; ++i) {
    const int r = h * d.B + i, a = row_ptr[r];
    if (row_has(col_idx + a, max(0, min(row_ptr[r + 1] - a, d.B)), j)) out[run++] = i;
  }
}

// ---------------------------------------------------------------------------
// Direct-to-LDS tile loads of NW waves through buffer resources.  A row tile
// (ROWS x 64 bf16) is ROWS*8 chunks, chunk (row, pc) filled from logical
// chunk pc ^ swz_k(row); a transposed tile (64 dims x 64 tokens) is 64*8
// chunks, chunk (dim, pc) from logical chunk pc ^ swz_v<64>(dim).  Load i of
// wave w fills the 64 chunks of block LPW w + i (rows or dims 8 blk .. 8 blk
// + 7); both swizzles depend on the block only through its parity, so two
// per-lane byte offsets per tile kind cover every load, and the block's
// position is a scalar offset.
struct TileOffsets {
  uint32_t row[2], col[2];
};
__device__ inline TileOffsets tile_offsets(int lane, uint32_t col_row_bytes) {
  TileOffsets o;
  const int r = lane >> 3, pc = lane & 7;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    o.row[j] = (uint32_t)(r * 128 + 16 * (pc ^ swz_k(8 * j + r)));
    o.col[j] = (uint32_t)r * col_row_bytes + 16 * (pc ^ swz_v<64>(8 * j + r));
  }
  return o;
}
// Fourth word of a raw buffer resource (byte addressing, 32-bit data format)
constexpr int kBufWord3 = 0x00020000;
__device__ inline __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufWord3);
}
template <int ROWS, int NW>
__device__ inline void load_rows(__amdgpu_buffer_rsrc_t rs, const TileOffsets& to, int row0,
                                 u32x4* lds, int w) {
  constexpr int LPW = ROWS * 8 / (64 * NW);
  static_assert(LPW >= 1 && (LPW == 1 || LPW % 2 == 0), "row tile loads");
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int blk = LPW * w + i;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)((lds_u32x4*)lds + blk * 64), 16,
                                             to.row[blk & 1], (row0 + 8 * blk) * 128, 0, 0);
  }
}
template <int NW>
__device__ inline void load_cols(__amdgpu_buffer_rsrc_t rs, const TileOffsets& to,
                                 uint32_t row_bytes, int col0, u32x4* lds, int w) {
  constexpr int LPW = 8 / NW;  // 64 dims x 8 chunks = 8 blocks of 64 chunks
  static_assert(LPW >= 1 && (LPW == 1 || LPW % 2 == 0), "column tile loads");
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int blk = LPW * w + i;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)((lds_u32x4*)lds + blk * 64), 16,
                                             to.col[blk & 1], 8 * blk * row_bytes + col0 * 2, 0, 0);
  }
}

// 32-token transposed tiles (64 dim rows of 4 chunks): chunk c of dim row r
// sits at c ^ swz_c32(r), which depends on bits 1-3 of r only, so that the
// operand reads of 8 and of 16 consecutive dim rows touch distinct banks.  A
// 64-lane load covers 16 dim rows, lane -> (row lane / 4, chunk lane % 4).
__device__ inline int swz_c32(int r) { return ((r >> 1) ^ ((r >> 3) & 1)) & 3; }
__device__ inline uint32_t col32_tile_offset(int lane, uint32_t col_row_bytes) {
  const int r = lane >> 2;
  return (uint32_t)r * col_row_bytes + 16 * ((lane & 3) ^ swz_c32(r));
}
template <int NW>
__device__ inline void load_cols32(__amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t row_bytes,
                                   int col0, u32x4* lds, int w) {
  constexpr int LPW = 4 / NW;  // 64 dims x 4 chunks = 4 blocks of 64 chunks
  static_assert(LPW >= 1, "column tile loads");
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int blk = LPW * w + i;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)((lds_u32x4*)lds + blk * 64), 16, off,
                                             16 * blk * row_bytes + col0 * 2, 0, 0);
  }
}
constexpr uint32_t kHalfCols32 = 32 * 4 * 16;  // 32 dims of a transposed 32-token tile, bytes

// Per-lane LDS byte offsets of the MFMA A operands within a tile: row tiles
// (K, V, Q, dO rows) at sub-tile 0 and k-step m, sub-tile t adding t * 32
// rows; transposed 64-token tiles at the tokens of (sub-tile t, half h2) for
// dims l32, dims 32 + l32 adding 32 rows.  With the tile's slot a
// compile-time constant every operand read is a base register plus an
// immediate offset.
struct OperandOffsets {
  uint32_t row[4], col[2][2];
};
__device__ inline OperandOffsets operand_offsets(int l32, int hh) {
  OperandOffsets o;
  const int R0 = pi_row(l32);
#pragma unroll
  for (int m = 0; m < 4; ++m) o.row[m] = (uint32_t)(R0 * 8 + ((4 * hh + m) ^ swz_k(R0))) * 16;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
      o.col[t][h2] = (uint32_t)(l32 * 8 + ((4 * t + 2 * h2 + hh) ^ swz_v<64>(l32))) * 16;
  return o;
}
constexpr uint32_t kSubRows = 32 * 8 * 16;   // 32 rows of a row tile, bytes
constexpr uint32_t kHalfCols = 32 * 8 * 16;  // 32 dims of a transposed 64-token tile, bytes
__device__ inline bf16x8 lds_op(const u32x4* smem, uint32_t off) {
  return as_bf16x8(*(const u32x4*)((const char*)smem + off));
}
__device__ inline f16x8 lds_op16(const u32x4* smem, uint32_t off) {
  return __builtin_bit_cast(f16x8, *(const u32x4*)((const char*)smem + off));
}
// Score r of a lane's 32-row sub-tile accumulator is row pi(8 (r / 4) + 4 hh
// + r % 4) = kc(r) + 8 hh of the sub-tile.
__device__ constexpr int acc_row(int r) { return 16 * (r >> 3) + 4 * ((r >> 2) & 1) + (r & 3); }

struct BwdArgs {
  const uint16_t* qp;   // packed rows
  const uint16_t* qt;   // packed transposed
  const uint16_t* dop;
  const uint16_t* dot;
  const uint16_t* kp;
  const uint16_t* kt;
  const uint16_t* vp;
  const float* lse2;    // [H][Ntot]
  const float* lse2s;   // [H][Ntot] lse2 - kPScaleLog2, read by dkdv_kernel
  const int* dosig;     // [H] sigma of the float16 dO^T copy
  const float* dd;      // [H][Ntot] D per packed row, read by dkdv_kernel
  float* dd_out;        // the same array, written by dq_kernel
  int d_given;          // D came from the float32 rows: dq_kernel skips its first sweep
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const int32_t* t_ptr;
  const int32_t* t_list;
  float* dq;            // [H][N][64] token order
  float* dk;
  float* dv;
  Dims d;
  int n_items;
};

// ---------------------------------------------------------------------------
// dQ: QT queries per workgroup (one patch block, or a tile of special
// queries), KT-key tiles: the kept blocks (TPB tiles each) then the special
// tiles for patch queries, every tile for special queries.
// 128-row workgroups take 64-key tiles and run three waves per SIMD (48 KB
// of LDS each, 159 VGPRs); 64-row workgroups (two waves) take 32-key tiles,
// whose 24 KB of LDS let four of them, two waves per SIMD, share a compute
// unit (64-key tiles would leave three).
template <int QT, int KT>
__global__ __launch_bounds__(2 * QT) __attribute__((amdgpu_waves_per_eu(QT == 128 ? 3 : 2,
                                                                         QT == 128 ? 3 : 2))) void dq_kernel(
    BwdArgs a) {
  constexpr int NW = QT / 32, NS = KT / 32, KCH = 8 * KT, TPB = QT / KT;
  static_assert(KT == 64 || KT == 32, "key tile");
  constexpr uint32_t kTile = KCH * 16;   // bytes of one tile
  __shared__ u32x4 smem[2 * 3 * KCH];  // slot s: K rows, V rows, K^T
  const Dims& d = a.d;
  const int item = __builtin_amdgcn_readfirstlane(xcd_item(wg_x(), a.n_items));
  if (item < 0) return;
  const int T = lid_x(), lane = T & 63;
  const int w = __builtin_amdgcn_readfirstlane(T >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int q_tiles = d.B + d.ns_pad / QT;
  const int h = __builtin_amdgcn_readfirstlane(item / q_tiles);
  const int qi = __builtin_amdgcn_readfirstlane(item - h * q_tiles);
  const bool patch_q = qi < d.B;
  const int qp0 = patch_q ? qi * QT : d.np_pad + (qi - d.B) * QT;
  int nt, nt_csr = 0;
  const int32_t* cols = nullptr;
  if (patch_q) {
    const int r0 = a.row_ptr[h * d.B + qi];
    cols = a.col_idx + r0;
    nt_csr = max(0, min(a.row_ptr[h * d.B + qi + 1] - r0, d.B));
    nt = nt_csr * TPB + d.ns_pad / KT;
  } else {
    nt = d.ntot_pad / KT;
  }
  nt = __builtin_amdgcn_readfirstlane(nt);
  nt_csr = __builtin_amdgcn_readfirstlane(nt_csr);
  auto tile_raw = [&](int n) -> int { return nt_csr > 0 ? cols[min(n / TPB, nt_csr - 1)] : 0; };
  auto tile_kp0 = [&](int n, int raw) -> int {
    raw = __builtin_amdgcn_readfirstlane(raw);
    if (!patch_q) return n * KT;
    const int nb = nt_csr * TPB;
    if (n >= nb) return d.np_pad + (n - nb) * KT;
    return min(max(raw, 0), d.B - 1) * QT + (n % TPB) * KT;
  };
  auto tile_valid = [&](int kp0) -> int {
    return kp0 < d.np_pad ? min(KT, d.np - kp0) : min(KT, d.ns - (kp0 - d.np_pad));
  };

  // this wave's 32 query rows: Q and dO fragments, lse2, D
  const int qrow = qp0 + 32 * w + l32;
  bf16x8 qop[4], dop[4];
  {
    const u32x4* sq = (const u32x4*)(a.qp + ((size_t)h * d.ntot_pad + qrow) * kHeadDim) + 4 * hh;
    const u32x4* so = (const u32x4*)(a.dop + ((size_t)h * d.ntot_pad + qrow) * kHeadDim) + 4 * hh;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      qop[m] = as_bf16x8(sq[m]);
      dop[m] = as_bf16x8(so[m]);
    }
  }
  const float lse2 = a.lse2[(size_t)h * d.ntot_pad + qrow];

  const uint32_t trow = (uint32_t)d.ntot_pad * 2;
  const uint32_t head_rows = (uint32_t)d.ntot_pad * 128;
  const __amdgpu_buffer_rsrc_t krs = buf_rsrc((const char*)a.kp + (size_t)h * head_rows, head_rows);
  const __amdgpu_buffer_rsrc_t vrs = buf_rsrc((const char*)a.vp + (size_t)h * head_rows, head_rows);
  const __amdgpu_buffer_rsrc_t ktrs = buf_rsrc((const char*)a.kt + (size_t)h * 64 * trow, 64 * trow);
  const TileOffsets to = tile_offsets(lane, trow);
  const OperandOffsets op = operand_offsets(l32, hh);
  // K^T operand chunks of dims l32 for sub-tile t, half h2 (add kHC for
  // dims 32 + l32)
  uint32_t colo[NS][2];
  constexpr uint32_t kHC = KT == 64 ? kHalfCols : kHalfCols32;
#pragma unroll
  for (int t = 0; t < NS; ++t)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
      colo[t][h2] = KT == 64 ? op.col[t][h2]
                             : (uint32_t)(4 * l32 + ((2 * h2 + hh) ^ swz_c32(l32))) * 16;
  const uint32_t to_c32 = KT == 32 ? col32_tile_offset(lane, trow) : 0u;
  auto issue = [&](int kp0, int slot, bool with_kt) {
    u32x4* base = smem + slot * 3 * KCH;
    load_rows<KT, NW>(krs, to, kp0, base, w);
    load_rows<KT, NW>(vrs, to, kp0, base + KCH, w);
    if (with_kt) {
      if constexpr (KT == 64) load_cols<NW>(ktrs, to, trow, kp0, base + 2 * KCH, w);
      else load_cols32<NW>(ktrs, to_c32, trow, kp0, base + 2 * KCH, w);
    }
  };

  // Two sweeps over the key tiles.  The first accumulates D = sum_k P dP,
  // which equals dO . O for this query, from the same float32 P and dP the
  // second sweep uses, so that the dS of a query sum to zero up to float32
  // rounding (D from the stored bf16 O would not, and the gradients of a
  // peaked softmax are exactly such small differences).  The second sweep
  // forms dS = P (dP - D) and feeds it to the dQ product as a bf16 pair
  // hi + lo (16 significant bits), for the same reason.  Tiles alternate
  // between two LDS slots; iterations come in pairs so the slot is a
  // compile-time constant.
  f32x16 g0 = {}, g1 = {};  // dQ^T: dims 0-31 and 32-63 x the wave's 32 queries
  float d_lane = 0.f, dq_d = 0.f;
  // each sweep is its own instance of the tile loop (its registers and
  // branches specialised to what it computes)
  auto sweep = [&](auto second_tag) {
    constexpr bool second = decltype(second_tag)::value;
    int raw_cur = tile_raw(0), raw_nxt = tile_raw(1);
    issue(tile_kp0(0, raw_cur), 0, second);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    auto step = [&](auto par, int n) {
      constexpr int P = decltype(par)::value;
      constexpr uint32_t kb = P * 3 * kTile, vb = kb + kTile, ktb = kb + 2 * kTile;
      if (n + 1 < nt) issue(tile_kp0(n + 1, raw_nxt), P ^ 1, second);
      const int raw_after = tile_raw(n + 2);
      const int valid = tile_valid(tile_kp0(n, raw_cur));
      // only a partial tile (the last patch block, the last special tile)
      // masks keys past its end; full tiles run the same code without it
      auto tile = [&](auto full_tag) {
        constexpr bool kFull = decltype(full_tag)::value;
        const int lim = valid - 8 * hh;  // key acc_row(r) + 8 hh of a sub-tile t is kept iff 32 t + acc_row(r) < lim
#pragma unroll
        for (int t = 0; t < NS; ++t) {
          f32x16 s = {}, dp = {};
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_op(smem, kb + op.row[m] + t * kSubRows),
                                                        qop[m], s, 0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_op(smem, vb + op.row[m] + t * kSubRows),
                                                         dop[m], dp, 0, 0, 0);
          }
          if constexpr (!second) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float p = fast_exp2(fmaf(s[r], kScaleLog2, -lse2));
              d_lane = fmaf((kFull || 32 * t + acc_row(r) < lim) ? p : 0.f, dp[r], d_lane);
            }
          } else {
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            f32x8 e8, rem;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int r = 8 * h2 + e;
              const float p = fast_exp2(fmaf(s[r], kScaleLog2, -lse2));
              e8[e] = (kFull || 32 * t + acc_row(r) < lim) ? p * (dp[r] - dq_d) : 0.f;
            }
            const bf16x8 ds_hi = __builtin_convertvector(e8, bf16x8);
#pragma unroll
            for (int e = 0; e < 8; ++e) rem[e] = e8[e] - (float)ds_hi[e];
            const bf16x8 ds_lo = __builtin_convertvector(rem, bf16x8);
            const bf16x8 k0 = lds_op(smem, ktb + colo[t][h2]);
            const bf16x8 k1 = lds_op(smem, ktb + colo[t][h2] + kHC);
            g0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, ds_hi, g0, 0, 0, 0);
            g1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, ds_hi, g1, 0, 0, 0);
            g0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, ds_lo, g0, 0, 0, 0);
            g1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, ds_lo, g1, 0, 0, 0);
          }
          }
        }
      };
      if (valid == KT) tile(std::true_type{});
      else tile(std::false_type{});
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      raw_cur = raw_nxt;
      raw_nxt = raw_after;
    };
    for (int n = 0;;) {
      step(std::integral_constant<int, 0>{}, n);
      if (++n == nt) break;
      step(std::integral_constant<int, 1>{}, n);
      if (++n == nt) break;
    }
    if constexpr (!second) {
      dq_d = xor32_sum(d_lane);  // lanes l and l + 32 hold the same query
      if (hh == 0) a.dd_out[(size_t)h * d.ntot_pad + qrow] = dq_d;
    }
  };
  if (nt > 0) {
    if (a.d_given)
      dq_d = a.dd[(size_t)h * d.ntot_pad + qrow];
    else
      sweep(std::false_type{});
    sweep(std::true_type{});
  }
  if (nt == 0 && hh == 0 && !a.d_given) a.dd_out[(size_t)h * d.ntot_pad + qrow] = 0.f;
  const int tok = packed_token(qrow, d);
  if (tok < 0) return;
  float* out = a.dq + ((size_t)h * d.n + tok) * kHeadDim;
#pragma unroll
  for (int aa = 0; aa < 4; ++aa) {
    *(f32x4*)(out + 8 * aa + 4 * hh) =
        f32x4{g0[4 * aa], g0[4 * aa + 1], g0[4 * aa + 2], g0[4 * aa + 3]} * 0.125f;
    *(f32x4*)(out + 32 + 8 * aa + 4 * hh) =
        f32x4{g1[4 * aa], g1[4 * aa + 1], g1[4 * aa + 2], g1[4 * aa + 3]} * 0.125f;
  }
}

// ---------------------------------------------------------------------------
// dK, dV: KT keys per workgroup (one patch block, or a tile of special keys),
// QT-query tiles: for a patch key block the query blocks that keep it (from
// the transposed CSR, qpb tiles each) then every special query tile; for
// special keys every query tile.  128-key workgroups take 64-query tiles;
// 64-key workgroups (two waves) take 32-query tiles, whose two 16 KB LDS
// slots let four workgroups, two waves per SIMD, share a compute unit
// (64-query tiles would leave one).
template <int KT, int QT>
__global__ __launch_bounds__(2 * KT) __attribute__((amdgpu_waves_per_eu(2, 2))) void dkdv_kernel(
    BwdArgs a, int qpb) {
  constexpr int NW = KT / 32, NS = QT / 32, QCH = 8 * QT;
  constexpr uint32_t kTile = QCH * 16;
  static_assert(QT == 64 || QT == 32, "query tile");
  static_assert(QT == 32 || NW >= 2, "one 64-lane load per statistics row");
  // slot s: Q rows, dO rows, Q^T, dO^T, then lse2 and D
  __shared__ u32x4 smem[2 * 4 * QCH];
  __shared__ float stats[2][2][QT];
  const Dims& d = a.d;
  const int item = __builtin_amdgcn_readfirstlane(xcd_item(wg_x(), a.n_items));
  if (item < 0) return;
  const int T = lid_x(), lane = T & 63;
  const int w = __builtin_amdgcn_readfirstlane(T >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int k_tiles = d.B + d.ns_pad / KT;
  const int h = __builtin_amdgcn_readfirstlane(item / k_tiles);
  const int kj = __builtin_amdgcn_readfirstlane(item - h * k_tiles);
  const bool patch_k = kj < d.B;
  const int kp0 = patch_k ? kj * KT : d.np_pad + (kj - d.B) * KT;
  int nt, nt_t = 0;
  const int32_t* qlist = nullptr;
  if (patch_k) {
    const int r0 = a.t_ptr[h * d.B + kj];
    qlist = a.t_list + r0;
    nt_t = max(0, min(a.t_ptr[h * d.B + kj + 1] - r0, d.B));
    nt = nt_t * qpb + d.ns_pad / QT;
  } else {
    nt = d.ntot_pad / QT;
  }
  nt = __builtin_amdgcn_readfirstlane(nt);
  nt_t = __builtin_amdgcn_readfirstlane(nt_t);
  auto tile_raw = [&](int n) -> int { return nt_t > 0 ? qlist[min(n / qpb, nt_t - 1)] : 0; };
  auto tile_qp0 = [&](int n, int raw) -> int {
    raw = __builtin_amdgcn_readfirstlane(raw);
    if (!patch_k) return n * QT;
    const int nb = nt_t * qpb;
    if (n >= nb) return d.np_pad + (n - nb) * QT;
    return min(max(raw, 0), d.B - 1) * (qpb * QT) + (n % qpb) * QT;
  };

  // this wave's 32 keys: K and V fragments
  const int krow = kp0 + 32 * w + l32;
  bf16x8 kop[4], vop[4];
  {
    const u32x4* sk = (const u32x4*)(a.kp + ((size_t)h * d.ntot_pad + krow) * kHeadDim) + 4 * hh;
    const u32x4* sv = (const u32x4*)(a.vp + ((size_t)h * d.ntot_pad + krow) * kHeadDim) + 4 * hh;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      kop[m] = as_bf16x8(sk[m]);
      vop[m] = as_bf16x8(sv[m]);
    }
  }

  const size_t hrow = (size_t)h * d.ntot_pad;
  const uint32_t trow = (uint32_t)d.ntot_pad * 2;
  const uint32_t head_rows = (uint32_t)d.ntot_pad * 128;
  const __amdgpu_buffer_rsrc_t qrs = buf_rsrc((const char*)a.qp + hrow * 128, head_rows);
  const __amdgpu_buffer_rsrc_t ors = buf_rsrc((const char*)a.dop + hrow * 128, head_rows);
  const __amdgpu_buffer_rsrc_t qtrs = buf_rsrc((const char*)a.qt + (size_t)h * 64 * trow, 64 * trow);
  const __amdgpu_buffer_rsrc_t otrs = buf_rsrc((const char*)a.dot + (size_t)h * 64 * trow, 64 * trow);
  const TileOffsets to = tile_offsets(lane, trow);
  const uint32_t to_c32 = QT == 32 ? col32_tile_offset(lane, trow) : 0u;
  const OperandOffsets op = operand_offsets(l32, hh);
  // Q^T, dO^T operand chunks of dims l32 for sub-tile t, half h2 (add
  // kHC for dims 32 + l32)
  uint32_t colo[NS][2];
  constexpr uint32_t kHC = QT == 64 ? kHalfCols : kHalfCols32;
#pragma unroll
  for (int t = 0; t < NS; ++t)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
      colo[t][h2] = QT == 64 ? op.col[t][h2]
                             : (uint32_t)(4 * l32 + ((2 * h2 + hh) ^ swz_c32(l32))) * 16;
  auto issue = [&](int qp0, int slot) {
    u32x4* base = smem + slot * 4 * QCH;
    load_rows<QT, NW>(qrs, to, qp0, base, w);
    load_rows<QT, NW>(ors, to, qp0, base + QCH, w);
    if constexpr (QT == 64) {
      load_cols<NW>(qtrs, to, trow, qp0, base + 2 * QCH, w);
      load_cols<NW>(otrs, to, trow, qp0, base + 3 * QCH, w);
      // lse2 and D of the tile's 64 queries: one 4-byte direct-to-LDS load
      // per lane, issued by waves 0 and 1 (no register round trip, no extra
      // wait)
      if (w < 2)
        __builtin_amdgcn_global_load_lds(
            (const void*)((w == 0 ? a.lse2s : a.dd) + hrow + qp0 + lane),
            (lds_void*)&stats[slot][w][0], 4, 0, 0);
    } else {
      load_cols32<NW>(qtrs, to_c32, trow, qp0, base + 2 * QCH, w);
      load_cols32<NW>(otrs, to_c32, trow, qp0, base + 3 * QCH, w);
      // lse2 (lanes 0-31) and D (lanes 32-63) of the tile's 32 queries from
      // wave 0: the two 32-float rows of stats[slot] are contiguous
      if (w == 0)
        __builtin_amdgcn_global_load_lds(
            (const void*)((hh ? a.dd : a.lse2s) + hrow + qp0 + l32),
            (lds_void*)&stats[slot][0][0], 4, 0, 0);
    }
  };

  // Query tiles alternate between two LDS slots; iterations come in pairs so
  // the slot is a compile-time constant.
  f32x16 v0 = {}, v1 = {}, k0 = {}, k1 = {};  // dV^T, dK^T: dims x the wave's 32 keys
  if (nt > 0) {
    int raw_cur = tile_raw(0), raw_nxt = tile_raw(1);
    issue(tile_qp0(0, raw_cur), 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    auto step = [&](auto par, int n) {
      constexpr int P = decltype(par)::value;
      constexpr uint32_t qb = P * 4 * kTile, ob = qb + kTile, qtb = qb + 2 * kTile, otb = qb + 3 * kTile;
      if (n + 1 < nt) issue(tile_qp0(n + 1, raw_nxt), P ^ 1);
      const int raw_after = tile_raw(n + 2);
      const float* lse_t = stats[P][0] + 8 * hh;
      const float* dd_t = stats[P][1] + 8 * hh;
#pragma unroll
      for (int t = 0; t < NS; ++t) {
        f32x16 s = {}, dp = {};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_op(smem, qb + op.row[m] + t * kSubRows),
                                                      kop[m], s, 0, 0, 0);
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_op(smem, ob + op.row[m] + t * kSubRows),
                                                       vop[m], dp, 0, 0, 0);
        }
        // accumulator entry r of this lane is query 32 t + acc_row(r) + 8 hh;
        // the exponential / product stretch runs at raised issue priority, as
        // in the forward (0.7 % faster here; the dQ kernel measured slower)
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          f32x8 p8, s8;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int r = 8 * h2 + e;
            const int qq = 32 * t + acc_row(r);
            const float p = fast_exp2(fmaf(s[r], kScaleLog2, -lse_t[qq]));
            p8[e] = p;
            s8[e] = p * (dp[r] - dd_t[qq]);
          }
          // P enters dV once as float16 (11 significant bits; a bf16
          // rounding of each weight would dominate the error of a key that
          // sums thousands of weighted rows), dS enters dK as a bf16 pair
          // hi + lo (dS is a small difference of large terms)
          const f16x8 pf = __builtin_convertvector(p8, f16x8);
          const bf16x8 sb = __builtin_convertvector(s8, bf16x8);
          f32x8 rem;
#pragma unroll
          for (int e = 0; e < 8; ++e) rem[e] = s8[e] - (float)sb[e];
          const bf16x8 sl = __builtin_convertvector(rem, bf16x8);
          const f16x8 o0 = lds_op16(smem, otb + colo[t][h2]);
          const f16x8 o1 = lds_op16(smem, otb + colo[t][h2] + kHC);
          const bf16x8 q0 = lds_op(smem, qtb + colo[t][h2]);
          const bf16x8 q1 = lds_op(smem, qtb + colo[t][h2] + kHC);
          v0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(o0, pf, v0, 0, 0, 0);
          v1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(o1, pf, v1, 0, 0, 0);
          k0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q0, sb, k0, 0, 0, 0);
          k1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q1, sb, k1, 0, 0, 0);
          k0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q0, sl, k0, 0, 0, 0);
          k1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q1, sl, k1, 0, 0, 0);
        }
        __builtin_amdgcn_s_setprio(0);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      raw_cur = raw_nxt;
      raw_nxt = raw_after;
    };
    for (int n = 0;;) {
      step(std::integral_constant<int, 0>{}, n);
      if (++n == nt) break;
      step(std::integral_constant<int, 1>{}, n);
      if (++n == nt) break;
    }
  }
  const int tok = packed_token(krow, d);
  if (tok < 0) return;
  float* ok = a.dk + ((size_t)h * d.n + tok) * kHeadDim;
  float* ov = a.dv + ((size_t)h * d.n + tok) * kHeadDim;
  // exact powers of two: 1/8 and 2^-15 for dK, 2^-(15 + sigma) for dV
  const float ks = __builtin_amdgcn_ldexpf(0.125f, -(int)kPScaleLog2);
  const float vs = __builtin_amdgcn_ldexpf(1.f, -(int)kPScaleLog2 - a.dosig[h]);
#pragma unroll
  for (int aa = 0; aa < 4; ++aa) {
    *(f32x4*)(ok + 8 * aa + 4 * hh) =
        f32x4{k0[4 * aa], k0[4 * aa + 1], k0[4 * aa + 2], k0[4 * aa + 3]} * ks;
    *(f32x4*)(ok + 32 + 8 * aa + 4 * hh) =
        f32x4{k1[4 * aa], k1[4 * aa + 1], k1[4 * aa + 2], k1[4 * aa + 3]} * ks;
    *(f32x4*)(ov + 8 * aa + 4 * hh) =
        f32x4{v0[4 * aa], v0[4 * aa + 1], v0[4 * aa + 2], v0[4 * aa + 3]} * vs;
    *(f32x4*)(ov + 32 + 8 * aa + 4 * hh) =
        f32x4{v1[4 * aa], v1[4 * aa + 1], v1[4 * aa + 2], v1[4 * aa + 3]} * vs;
  }
}

// ---------------------------------------------------------------------------
size_t backward_workspace(const Dims& d) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t arr = up((size_t)d.H * d.ntot_pad * kHeadDim * sizeof(uint16_t));
  return 7 * arr + 3 * up((size_t)d.H * d.ntot_pad * sizeof(float)) +
         up((size_t)d.H * kAbsmaxChunks * sizeof(uint32_t)) +  // dO chunk maxima
         up((size_t)d.H * sizeof(int)) +                      // dO sigma
         up(((size_t)d.H * d.B + 1) * sizeof(int32_t)) +   // t_ptr
         up((size_t)d.H * d.B * sizeof(int32_t)) +         // counts
         up((size_t)d.H * d.B * d.B * sizeof(int32_t));   // t_list
}

hipError_t launch_scan_counts(const int32_t* counts, int rows, int32_t* row_ptr, hipStream_t st);

hipError_t launch_backward(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const uint16_t* o, const float* o32, const float* lse,
                           const uint16_t* d_o, const int32_t* row_ptr, const int32_t* col_idx,
                           float* dq, float* dk, float* dv, void* ws, hipStream_t st) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t arr = up((size_t)d.H * d.ntot_pad * kHeadDim * sizeof(uint16_t));
  char* p = (char*)ws;
  uint16_t* qp = (uint16_t*)p; p += arr;
  uint16_t* qt = (uint16_t*)p; p += arr;
  uint16_t* dop = (uint16_t*)p; p += arr;
  uint16_t* dot = (uint16_t*)p; p += arr;
  uint16_t* kp = (uint16_t*)p; p += arr;
  uint16_t* kt = (uint16_t*)p; p += arr;
  uint16_t* vp = (uint16_t*)p; p += arr;
  float* lse2 = (float*)p; p += up((size_t)d.H * d.ntot_pad * sizeof(float));
  float* lse2s = (float*)p; p += up((size_t)d.H * d.ntot_pad * sizeof(float));
  float* dd = (float*)p; p += up((size_t)d.H * d.ntot_pad * sizeof(float));
  uint32_t* do_max = (uint32_t*)p; p += up((size_t)d.H * kAbsmaxChunks * sizeof(uint32_t));
  int* dosig = (int*)p; p += up((size_t)d.H * sizeof(int));
  int32_t* t_ptr = (int32_t*)p; p += up(((size_t)d.H * d.B + 1) * sizeof(int32_t));
  int32_t* counts = (int32_t*)p; p += up((size_t)d.H * d.B * sizeof(int32_t));
  int32_t* t_list = (int32_t*)p;

  const dim3 pg(d.ntot_pad / 64, d.H);
  const int nchunk = absmax_chunks(d);
  hipError_t e = launch_absmax(d, d_o, do_max, st);
  if (e != hipSuccess) return e;
  bwd_pack_kernel<<<pg, 256, 0, st>>>((const uint4*)q, (uint4*)qp, (uint4*)qt, d, nullptr,
                                      nullptr, 0);
  bwd_pack_kernel<<<pg, 256, 0, st>>>((const uint4*)d_o, (uint4*)dop, (uint4*)dot, d, do_max,
                                      dosig, nchunk);
  bwd_pack_kernel<<<pg, 256, 0, st>>>((const uint4*)k, (uint4*)kp, (uint4*)kt, d, nullptr,
                                      nullptr, 0);
  bwd_pack_kernel<<<pg, 256, 0, st>>>((const uint4*)v, (uint4*)vp, nullptr, d, nullptr, nullptr,
                                      0);
  bwd_rowstats_kernel<<<dim3(d.ntot_pad / 32, d.H), 256, 0, st>>>(
      (const uint4*)o, (const float4*)o32, (const uint4*)d_o, lse, lse2, lse2s, dd, d);
  csr_t_count_kernel<<<dim3(d.B, d.H), 256, 0, st>>>(row_ptr, col_idx, d, counts);
  e = launch_scan_counts(counts, d.H * d.B, t_ptr, st);
  if (e != hipSuccess) return e;
  csr_t_fill_kernel<<<dim3(d.B, d.H), 256, 0, st>>>(row_ptr, col_idx, t_ptr, d, t_list);

  BwdArgs a = {};
  a.qp = qp; a.qt = qt; a.dop = dop; a.dot = dot; a.kp = kp; a.kt = kt; a.vp = vp;
  a.lse2 = lse2; a.lse2s = lse2s; a.dosig = dosig; a.dd = dd; a.dd_out = dd;
  a.d_given = o32 != nullptr; a.row_ptr = row_ptr; a.col_idx = col_idx;
  a.t_ptr = t_ptr; a.t_list = t_list; a.dq = dq; a.dk = dk; a.dv = dv; a.d = d;
  if (d.b == 128) {
    a.n_items = d.H * (d.B + d.ns_pad / 128);
    dq_kernel<128, 64><<<xcd_grid(a.n_items), 256, 0, st>>>(a);
    a.n_items = d.H * (d.B + d.ns_pad / 128);
    dkdv_kernel<128, 64><<<xcd_grid(a.n_items), 256, 0, st>>>(a, 2);
  } else {
    a.n_items = d.H * (d.B + d.ns_pad / 64);
    dq_kernel<64, 32><<<xcd_grid(a.n_items), 128, 0, st>>>(a);
    a.n_items = d.H * (d.B + d.ns_pad / 64);
    dkdv_kernel<64, 32><<<xcd_grid(a.n_items), 128, 0, st>>>(a, 2);
  }
  return hipGetLastError();
}

}  // namespace bsga
