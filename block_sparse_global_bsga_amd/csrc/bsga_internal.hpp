// Internal declarations shared by the libbsga HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/bsga.h"

namespace bsga {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kHeadDim = 64;
constexpr int kPad = 128;  // packed segments are padded to this many keys

// Exact unsigned division by a runtime constant (round-up multiplier method
// of Granlund & Montgomery, "Division by invariant integers using
// multiplication", 1994): q = (mulhi(n, m) + n) >> l, valid for every
// 32-bit n.
struct FastDiv {
  uint32_t d, m, l;
};

inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t l = 0;
  while (l < 32 && (uint64_t(1) << l) < d) ++l;
  f.l = l;
  f.m = (uint32_t)(((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1);
  return f;
}

__host__ __device__ inline uint32_t fdiv(uint32_t n, const FastDiv& f) {
  const uint32_t t = (uint32_t)(((uint64_t)n * f.m) >> 32);  // v_mul_hi_u32 on the device
  return (uint32_t)(((uint64_t)t + n) >> f.l);
}

// Workgroup and work-item ids straight from the hardware registers.  The
// attention and backward kernels are compiled without IEEE mode (their max
// chains never see NaNs), which keeps the device library's id functions from
// being inlined into them; the builtins need no call.
__device__ inline int wg_x() { return (int)__builtin_amdgcn_workgroup_id_x(); }
__device__ inline int wg_y() { return (int)__builtin_amdgcn_workgroup_id_y(); }
__device__ inline int lid_x() { return (int)__builtin_amdgcn_workitem_id_x(); }

// Layer geometry.  "Packed order" lists keys (and queries) as the N_p patch
// tokens in patch order, zero padding up to np_pad, then the N_s special
// tokens, padding up to np_pad + ns_pad.  Both pads are multiples of kPad.
struct Dims {
  int F, P, S, H, b, B;
  int np, ns, n;
  int np_pad, ns_pad, ntot_pad;
  FastDiv divP, divS;
};

Dims make_dims(const bsga_shape& s);

// Token row of patch p and of special token s.
__device__ inline uint32_t patch_token(uint32_t p, const Dims& d) {
  uint32_t f = fdiv(p, d.divP);
  return f * (uint32_t)(d.P + d.S) + (uint32_t)d.S + (p - f * (uint32_t)d.P);
}
__device__ inline uint32_t special_token(uint32_t s, const Dims& d) {
  uint32_t f = fdiv(s, d.divS);
  return f * (uint32_t)(d.P + d.S) + (s - f * (uint32_t)d.S);
}

// Token row of packed index kp, or -1 for padding.
__device__ inline int packed_token(int kp, const Dims& d) {
  if (kp < d.np_pad) return kp < d.np ? (int)patch_token(kp, d) : -1;
  int s = kp - d.np_pad;
  return s < d.ns ? (int)special_token(s, d) : -1;
}

// XCD-aware work mapping: the hardware deals workgroup ids round-robin over
// the 8 XCDs; give each XCD one contiguous range of work items so that
// neighbouring items (same head, nearby query blocks) share that XCD's L2.
// The grid must hold 8 * ceil(n / 8) workgroups; ids mapped past n return -1.
constexpr int kXcds = 8;
__device__ inline int xcd_item(int id, int n) {
  int per = (n + kXcds - 1) / kXcds;
  int item = (id % kXcds) * per + id / kXcds;
  return item < n ? item : -1;
}
inline int xcd_grid(int n) { return ((n + kXcds - 1) / kXcds) * kXcds; }

__device__ inline float xor32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                            __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float xor32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                            __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// Power-of-two operand scales.  An operand headed for a float16 MFMA operand
// is stored as x * 2^sigma, with sigma chosen per head from the head's
// largest |x| (bf16 bits with the sign cleared, mb) so that it lies in
// [2^14, 2^15): every bf16 value is then exact in float16 except those more
// than 2^28 below the maximum (float16 subnormals, absolute error under 2^-39
// of it).  sigma is clamped to [-100, 100]; 0 when the head has no finite
// nonzero value.  The maxima come per chunk of tokens (at most
// kAbsmaxChunks chunks per head) from launch_absmax.
constexpr int kAbsmaxChunks = 64;
inline int absmax_chunks(const Dims& d) {
  const int c = (d.n + 1023) / 1024;
  return c < kAbsmaxChunks ? c : kAbsmaxChunks;
}
__device__ inline int sigma_of_max(uint32_t mb) {
  if (mb == 0 || mb >= 0x7f80u) return 0;  // all zero, or inf / NaN present
  const int e = (int)(mb >> 7) - 127;      // max in [2^e, 2^(e+1)) (e = -127: subnormal)
  return min(100, max(-100, 14 - e));
}
// the largest |x| of head h from its chunk maxima, reduced by the 64 lanes
// of a wave (lane = the calling lane), as sigma
__device__ inline int head_sigma(const uint32_t* chunk_max, int h, int nchunk, int lane) {
  uint32_t m = lane < nchunk ? chunk_max[h * kAbsmaxChunks + lane] : 0u;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  return sigma_of_max(m);
}

// ---------------------------------------------------------------- launchers
// per (head, chunk) largest |x| of a [H][N][64] bf16 tensor, as bf16 bits,
// into chunk_max[H][kAbsmaxChunks]
hipError_t launch_absmax(const Dims& d, const uint16_t* x, uint32_t* chunk_max, hipStream_t st);
// Each returns hipSuccess or the launch error.  All pointers are device
// pointers validated by the caller.
hipError_t launch_pool(const Dims& d, const uint16_t* q, const uint16_t* k,
                       float* qbar, float* kbar, hipStream_t st);
hipError_t launch_scores(const Dims& d, const float* qbar, const float* kbar,
                         float* probs, float* scores, hipStream_t st);
hipError_t launch_softmax(const Dims& d, float* probs, hipStream_t st);

struct SelectParams {
  int k[BSGA_MAX_HEADS];
  double tau;
};
size_t select_workspace(const Dims& d);
hipError_t launch_select(const Dims& d, const float* probs,
                         const SelectParams& sp, int32_t* row_ptr,
                         int32_t* col_idx, void* ws, hipStream_t st);

// device address and size of the selection scratch array of the current
// device (bsga_select_static)
hipError_t select_static_scratch(void** out, size_t* bytes);

size_t probe_workspace(const Dims& d);
hipError_t launch_probe_select(const Dims& d, const uint16_t* q, const uint16_t* k, int topk,
                               float* scores, int32_t* row_ptr, int32_t* col_idx, void* ws,
                               hipStream_t st);

size_t nmse_workspace(const Dims& d);
hipError_t launch_nmse(const Dims& d, const uint16_t* ref, const uint16_t* out, double* result,
                       void* ws, hipStream_t st);

size_t backward_workspace(const Dims& d);
// Exactly one of o (the bf16 rows; D = sum_k P dP is then recomputed by
// dq_kernel) and o32 (float32 rows from the training-mode forward; D = dO . O
// from them, and dq_kernel runs its gradient sweep only) is non-null.
hipError_t launch_backward(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const uint16_t* o, const float* o32, const float* lse,
                           const uint16_t* d_o, const int32_t* row_ptr, const int32_t* col_idx,
                           float* dq, float* dk, float* dv, void* ws, hipStream_t st);

size_t pack_bytes(const Dims& d);  // packed K and V^T
hipError_t launch_pack(const Dims& d, const uint16_t* k, const uint16_t* v,
                       uint16_t* kp, uint16_t* vt, hipStream_t st);
hipError_t launch_sparse_attn(const Dims& d, const uint16_t* q,
                              const uint16_t* kp, const uint16_t* vt,
                              const int32_t* row_ptr, const int32_t* col_idx,
                              uint16_t* o, float* lse, hipStream_t st);
// ws (optional, patch_rows_workspace bytes): lets b = 128 rows of the last,
// partial round of workgroups run as key-range pieces merged afterwards
size_t patch_rows_workspace(const Dims& d);
// o32 (training mode, needs ws; b = 128 or b = 64 with B <= 8192): P enters
// P V as a float16 pair hi + lo and the final rows are also written as
// float32 [H][N][64]
hipError_t launch_patch_rows(const Dims& d, const uint16_t* q, const uint16_t* kp,
                             const uint16_t* vt, const int32_t* row_ptr, const int32_t* col_idx,
                             uint16_t* o, float* lse, hipStream_t st, void* ws = nullptr,
                             size_t ws_bytes = 0, float* o32 = nullptr);
bool patch_rows_train_supported(const Dims& d);
size_t special_workspace(const Dims& d);
hipError_t launch_special_rows(const Dims& d, const uint16_t* q, const uint16_t* kp,
                               const uint16_t* vt, uint16_t* o, float* lse, void* ws,
                               hipStream_t st, float* o32 = nullptr);
hipError_t launch_special(const Dims& d, const uint16_t* q,
                          const uint16_t* kp, const uint16_t* vt, uint16_t* o,
                          float* lse, void* ws, hipStream_t st);
hipError_t launch_dense(const Dims& d, const uint16_t* q, const uint16_t* kp,
                        const uint16_t* vt, uint16_t* o, float* lse,
                        hipStream_t st);

}  // namespace bsga
