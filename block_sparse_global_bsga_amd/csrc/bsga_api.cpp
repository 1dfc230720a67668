// C ABI of libbsga: argument validation (before anything is enqueued),
// exact host integers (B, k_h), workspace carving and kernel launches.
#include <math.h>
#include <string.h>

#include "bsga_internal.hpp"

namespace bsga {

Dims make_dims(const bsga_shape& s) {
  Dims d;
  d.F = s.frames;
  d.P = s.patches_per_frame;
  d.S = s.special_per_frame;
  d.H = s.heads;
  d.b = s.block;
  d.np = d.F * d.P;
  d.ns = d.F * d.S;
  d.n = d.np + d.ns;
  d.B = (d.np + d.b - 1) / d.b;
  d.np_pad = (d.np + kPad - 1) / kPad * kPad;
  d.ns_pad = (d.ns + kPad - 1) / kPad * kPad;
  d.ntot_pad = d.np_pad + d.ns_pad;
  d.divP = make_fastdiv((uint32_t)d.P);
  d.divS = make_fastdiv((uint32_t)(d.S > 0 ? d.S : 1));
  return d;
}

}  // namespace bsga

using namespace bsga;

namespace {

constexpr size_t kAlign = 256;
inline size_t up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

int check_shape(const bsga_shape* s) {
  if (!s) return BSGA_ERR_INVALID_ARG;
  if (s->frames < 1 || s->patches_per_frame < 1 || s->special_per_frame < 0 || s->heads < 1)
    return BSGA_ERR_INVALID_ARG;
  if (s->head_dim != kHeadDim) return BSGA_ERR_UNSUPPORTED;
  if (s->block != 64 && s->block != 128) return BSGA_ERR_UNSUPPORTED;
  // 32-bit byte offsets within one head inside the kernels: a head's padded
  // [tokens][64] bf16 array must stay below 2 GB (about 16.7 million tokens)
  const int64_t n = (int64_t)s->frames * ((int64_t)s->patches_per_frame + s->special_per_frame);
  const int64_t npad = n + 2 * kPad;
  if (npad * kHeadDim * 2 >= ((int64_t)1 << 31)) return BSGA_ERR_UNSUPPORTED;
  const int64_t np = (int64_t)s->frames * s->patches_per_frame;
  const int64_t B = (np + s->block - 1) / s->block;
  if ((int64_t)s->heads * B >= ((int64_t)1 << 31)) return BSGA_ERR_UNSUPPORTED;
  return BSGA_OK;
}

// CSR-producing calls also need H*B*B to fit int32 and B within the sort.
int check_select_shape(const Dims& d) {
  if (d.B > BSGA_MAX_BLOCKS) return BSGA_ERR_UNSUPPORTED;
  if ((int64_t)d.H * d.B * d.B >= ((int64_t)1 << 31)) return BSGA_ERR_UNSUPPORTED;
  if (d.H > BSGA_MAX_HEADS) return BSGA_ERR_UNSUPPORTED;
  return BSGA_OK;
}

int check_ptr(const void* p, size_t align) {
  if (!p) return BSGA_ERR_INVALID_ARG;
  if ((uintptr_t)p % align) return BSGA_ERR_MISALIGNED;
  return BSGA_OK;
}

bool bad_prob(double x) { return !(x >= 0.0 && x <= 1.0); }  // also NaN

int exact_keep(int32_t B, double rho) {
  const int64_t r = (int64_t)nearbyint(rho * 1e6);
  return (int)(((int64_t)B * (1000000 - r)) / 1000000);
}

size_t ws_predict(const Dims& d) { return 2 * up((size_t)d.H * d.B * kHeadDim * sizeof(float)); }
size_t ws_select(const Dims& d) { return up(select_workspace(d)); }
size_t ws_pack(const Dims& d) { return up(pack_bytes(d)); }
size_t ws_special(const Dims& d) { return up(special_workspace(d)); }
size_t ws_probe(const Dims& d) { return up(probe_workspace(d)); }
size_t ws_nmse(const Dims& d) { return up(nmse_workspace(d)); }
size_t ws_backward(const Dims& d) { return up(backward_workspace(d)); }
size_t ws_patch_rows(const Dims& d) { return up(patch_rows_workspace(d)); }

size_t ws_for(const Dims& d, int op) {
  switch (op) {
    case BSGA_OP_PREDICT_MASK: return ws_predict(d);
    case BSGA_OP_SELECT: return ws_select(d);
    case BSGA_OP_SPARSE_ATTN: return ws_pack(d);
    case BSGA_OP_SPECIAL_DENSE: return ws_pack(d) + ws_special(d);
    case BSGA_OP_DENSE_ATTN: return ws_pack(d);
    case BSGA_OP_SPECIAL_DENSE_PACKED: return ws_special(d);
    case BSGA_OP_PROBE_SELECT: return ws_probe(d);
    case BSGA_OP_NMSE: return ws_nmse(d);
    case BSGA_OP_BACKWARD: return ws_backward(d);
    case BSGA_OP_PATCH_ROWS_PACKED: return ws_patch_rows(d);
    case BSGA_OP_LAYER: {
      size_t m = ws_predict(d);
      if (ws_select(d) > m) m = ws_select(d);
      if (ws_special(d) > m) m = ws_special(d);
      if (ws_patch_rows(d) > m) m = ws_patch_rows(d);
      return ws_pack(d) + m;
    }
    default: return 0;
  }
}

int check_ws(const Dims& d, int op, const void* ws, size_t bytes) {
  const size_t need = ws_for(d, op);
  if (need == 0) return BSGA_OK;
  if (!ws || ((uintptr_t)ws % kAlign) || bytes < need) return BSGA_ERR_WORKSPACE;
  return BSGA_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? BSGA_OK : BSGA_ERR_HIP; }

#define BSGA_TRY(x)                 \
  do {                              \
    const int _s = (x);             \
    if (_s != BSGA_OK) return _s;   \
  } while (0)

int fill_select_params(const Dims& d, const double* rho_per_head, double rho, double tau,
                       SelectParams* sp) {
  if (bad_prob(rho) || isnan(tau)) return BSGA_ERR_INVALID_ARG;
  if (rho_per_head)
    for (int h = 0; h < d.H; ++h)
      if (bad_prob(rho_per_head[h])) return BSGA_ERR_INVALID_ARG;
  memset(sp, 0, sizeof(*sp));
  for (int h = 0; h < d.H; ++h) sp->k[h] = exact_keep(d.B, rho_per_head ? rho_per_head[h] : rho);
  sp->tau = tau;
  return BSGA_OK;
}

int check_qk(const uint16_t* q, const uint16_t* k) {
  BSGA_TRY(check_ptr(q, 16));
  return check_ptr(k, 16);
}

int check_qkv(const uint16_t* q, const uint16_t* k, const uint16_t* v) {
  BSGA_TRY(check_qk(q, k));
  return check_ptr(v, 16);
}

int check_csr(const Dims& d, const int32_t* row_ptr, const int32_t* col_idx, int64_t cap) {
  BSGA_TRY(check_ptr(row_ptr, 4));
  BSGA_TRY(check_ptr(col_idx, 4));
  if (cap < (int64_t)d.H * d.B * d.B) return BSGA_ERR_INVALID_ARG;
  return BSGA_OK;
}

int check_packed(const Dims& d, const void* kv, size_t bytes) {
  if (!kv) return BSGA_ERR_INVALID_ARG;
  if ((uintptr_t)kv % kAlign) return BSGA_ERR_MISALIGNED;
  if (bytes < ws_pack(d)) return BSGA_ERR_INVALID_ARG;
  return BSGA_OK;
}

}  // namespace

extern "C" {

int bsga_version(void) { return BSGA_VERSION; }

const char* bsga_status_string(int status) {
  switch (status) {
    case BSGA_OK: return "ok";
    case BSGA_ERR_INVALID_ARG: return "invalid argument";
    case BSGA_ERR_UNSUPPORTED: return "unsupported shape or parameter";
    case BSGA_ERR_MISALIGNED: return "misaligned pointer";
    case BSGA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case BSGA_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int bsga_num_blocks(const bsga_shape* shape, int32_t* n_blocks) {
  BSGA_TRY(check_shape(shape));
  if (!n_blocks) return BSGA_ERR_INVALID_ARG;
  *n_blocks = make_dims(*shape).B;
  return BSGA_OK;
}

int bsga_keep_count(int32_t n_blocks, double rho, int32_t* k) {
  if (!k || n_blocks < 0 || bad_prob(rho)) return BSGA_ERR_INVALID_ARG;
  *k = exact_keep(n_blocks, rho);
  return BSGA_OK;
}

int bsga_csr_capacity(const bsga_shape* shape, int64_t* entries) {
  BSGA_TRY(check_shape(shape));
  if (!entries) return BSGA_ERR_INVALID_ARG;
  const Dims d = make_dims(*shape);
  *entries = (int64_t)d.H * d.B * d.B;
  return BSGA_OK;
}

int bsga_workspace_bytes(const bsga_shape* shape, int op, size_t* bytes) {
  BSGA_TRY(check_shape(shape));
  if (!bytes || op < BSGA_OP_PREDICT_MASK || op > BSGA_OP_PATCH_ROWS_PACKED)
    return BSGA_ERR_INVALID_ARG;
  *bytes = ws_for(make_dims(*shape), op);
  return BSGA_OK;
}

int bsga_predict_mask(const bsga_shape* shape, const uint16_t* q, const uint16_t* k, float* probs,
                      float* scores, float* qbar, float* kbar, void* ws, size_t ws_bytes,
                      void* stream) {
  BSGA_TRY(check_shape(shape));
  const Dims d = make_dims(*shape);
  BSGA_TRY(check_qk(q, k));
  BSGA_TRY(check_ptr(probs, 4));
  if (scores) BSGA_TRY(check_ptr(scores, 4));
  if (scores == probs) return BSGA_ERR_INVALID_ARG;
  if (qbar) BSGA_TRY(check_ptr(qbar, 4));
  if (kbar) BSGA_TRY(check_ptr(kbar, 4));
  BSGA_TRY(check_ws(d, BSGA_OP_PREDICT_MASK, ws, ws_bytes));
  const size_t half = up((size_t)d.H * d.B * kHeadDim * sizeof(float));
  float* qb = qbar ? qbar : (float*)ws;
  float* kb = kbar ? kbar : (float*)((char*)ws + half);
  hipStream_t st = (hipStream_t)stream;
  BSGA_TRY(hip_status(launch_pool(d, q, k, qb, kb, st)));
  BSGA_TRY(hip_status(launch_scores(d, qb, kb, probs, scores, st)));
  return hip_status(launch_softmax(d, probs, st));
}

int bsga_select(const bsga_shape* shape, const float* probs, const double* rho_per_head,
                double rho, double tau, int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                void* ws, size_t ws_bytes, void* stream) {
  BSGA_TRY(check_shape(shape));
  const Dims d = make_dims(*shape);
  BSGA_TRY(check_select_shape(d));
  BSGA_TRY(check_ptr(probs, 4));
  BSGA_TRY(check_csr(d, row_ptr, col_idx, col_capacity));
  SelectParams sp;
  BSGA_TRY(fill_select_params(d, rho_per_head, rho, tau, &sp));
  BSGA_TRY(check_ws(d, BSGA_OP_SELECT, ws, ws_bytes));
  return hip_status(launch_select(d, probs, sp, row_ptr, col_idx, ws, (hipStream_t)stream));
}

int bsga_select_static(const bsga_shape* shape, const float* probs, const double* rho_per_head,
                       double rho, double tau, int32_t* row_ptr, int32_t* col_idx,
                       int64_t col_capacity, void* stream) {
  BSGA_TRY(check_shape(shape));
  const Dims d = make_dims(*shape);
  BSGA_TRY(check_select_shape(d));
  if ((int64_t)d.H * d.B > BSGA_SELECT_STATIC_MAX_ROWS) return BSGA_ERR_UNSUPPORTED;
  BSGA_TRY(check_ptr(probs, 4));
  BSGA_TRY(check_csr(d, row_ptr, col_idx, col_capacity));
  SelectParams sp;
  BSGA_TRY(fill_select_params(d, rho_per_head, rho, tau, &sp));
  void* scratch = nullptr;
  size_t scratch_bytes = 0;
  BSGA_TRY(hip_status(select_static_scratch(&scratch, &scratch_bytes)));
  if (ws_select(d) > scratch_bytes) return BSGA_ERR_UNSUPPORTED;
  return hip_status(launch_select(d, probs, sp, row_ptr, col_idx, scratch, (hipStream_t)stream));
}

int bsga_probe_select(const bsga_shape* shape, const uint16_t* q, const uint16_t* k, int32_t topk,
                      float* scores, int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                      void* ws, size_t ws_bytes, void* stream) {
  BSGA_TRY(check_shape(shape));
  const Dims d = make_dims(*shape);
  BSGA_TRY(check_select_shape(d));
  BSGA_TRY(check_qk(q, k));
  if (topk < 0) return BSGA_ERR_INVALID_ARG;
  if (scores && ((uintptr_t)scores % 4)) return BSGA_ERR_MISALIGNED;
  BSGA_TRY(check_csr(d, row_ptr, col_idx, col_capacity));
  BSGA_TRY(check_ws(d, BSGA_OP_PROBE_SELECT, ws, ws_bytes));
  return hip_status(launch_probe_select(d, q, k, topk, scores, row_ptr, col_idx, ws,
                                        (hipStream_t)stream));
}

int bsga_nmse(const bsga_shape* shape, const uint16_t* o_ref, const uint16_t* o, double* nmse,
              void* ws, size_t ws_bytes, void* stream) {
  BSGA_TRY(check_shape(shape));
  const Dims d = make_dims(*shape);
  BSGA_TRY(check_ptr(o_ref, 16));
  BSGA_TRY(check_ptr(o, 16));
  BSGA_TRY(check_ptr(nmse, 8));
  BSGA_TRY(check_ws(d, BSGA_OP_NMSE, ws, ws_bytes));
  return hip_status(launch_nmse(d, o_ref, o, nmse, ws, (hipStream_t)stream));
}

int bsga_attn_backward(const bsga_shape* shape, const uint16_t* q, const uint16_t* k,
                       const uint16_t* v, const uint16_t* o, const float* lse,
                       const uint16_t* d_o, const int32_t* row_ptr, const int32_t* col_idx,
                       float* dq, float* dk, float* dv, void* ws, size_t ws_bytes, void* stream) {
  BSGA_TRY(check_shape(shape));
  const Dims d = make_dims(*shape);
  BSGA_TRY(check_select_shape(d));
  BSGA_TRY(check_qkv(q, k, v));
  BSGA_TRY(check_ptr(o, 16));
  BSGA_TRY(check_ptr(d_o, 16));
  BSGA_TRY(check_ptr(lse, 4));
  BSGA_TRY(check_ptr(row_ptr, 4));
  BSGA_TRY(check_ptr(col_idx, 4));
  BSGA_TRY(check_ptr(dq, 16));
  BSGA_TRY(check_ptr(dk, 16));
  BSGA_TRY(check_ptr(dv, 16));
  BSGA_TRY(check_ws(d, BSGA_OP_BACKWARD, ws, ws_bytes));
  return hip_status(launch_backward(d, q, k, v, o, nullptr, lse, d_o, row_ptr, col_idx, dq, dk,
                                    dv, ws, (hipStream_t)stream));
}

int bsga_attn_backward_o32(const bsga_shape* shape, const uint16_t* q, const uint16_t* k,
                           const uint16_t* v, const float* o32, const float* lse,
                           const uint16_t* d_o, const int32_t* row_ptr, const int32_t* col_idx,
                           float* dq, float* dk, float* dv, void* ws, size_t ws_bytes,
                           void* stream) {
  BSGA_TRY(check_shape(shape));
  const Dims d = make_dims(*shape);
  BSGA_TRY(check_select_shape(d));
  BSGA_TRY(check_qkv(q, k, v));
  BSGA_TRY(check_ptr(o32, 16));
  BSGA_TRY(check_ptr(d_o, 16));
  BSGA_TRY(check_ptr(lse, 4));
  BSGA_TRY(check_ptr(row_ptr, 4));
  BSGA_TRY(check_ptr(col_idx, 4));
  BSGA_TRY(check_ptr(dq, 16));
  BSGA_TRY(check_ptr(dk, 16));
  BSGA_TRY(check_ptr(dv, 16));
  BSGA_TRY(check_ws(d, BSGA_OP_BACKWARD, ws, ws_bytes));
  return hip_status(launch_backward(d, q, k, v, nullptr, o32, lse, d_o, row_ptr, col_idx, dq, dk,
                                    dv, ws, (hipStream_t)stream));
}

int bsga_sparse_attn(const bsga_shape* shape, const uint16_t* q, const uint16_t* k,
                     const uint16_t* v, const int32_t* row_ptr, const int32_t* col_idx,
                     uint16_t* o, float* lse, void* ws, size_t ws_bytes, void* stream) {
  BSGA_TRY(check_shape(shape));
  const Dims d = make_dims(*shape);
  BSGA_TRY(check_qkv(q, k, v));
  BSGA_TRY(check_ptr(row_ptr, 4));
  BSGA_TRY(check_ptr(col_idx, 4));
  BSGA_TRY(check_ptr(o, 16));
  BSGA_TRY(check_ptr(lse, 4));
  BSGA_TRY(check_ws(d, BSGA_OP_SPARSE_ATTN, ws, ws_bytes));
  hipStream_t st = (hipStream_t)stream;
  uint16_t* kp = (uint16_t*)ws;
  uint16_t* vt = kp + (size_t)d.H * d.ntot_pad * kHeadDim;
  BSGA_TRY(hip_status(launch_pack(d, k, v, kp, vt, st)));
  return hip_status(launch_sparse_attn(d, q, kp, vt, row_ptr, col_idx, o, lse, st));
}

int bsga_special_dense(const bsga_shape* shape, const uint16_t* q, const uint16_t* k,
                       const uint16_t* v, uint16_t* o, float* lse, void* ws, size_t ws_bytes,
                       void* stream) {
  BSGA_TRY(check_shape(shape));
  const Dims d = make_dims(*shape);
  BSGA_TRY(check_qkv(q, k, v));
  BSGA_TRY(check_ptr(o, 16));
  BSGA_TRY(check_ptr(lse, 4));
  BSGA_TRY(check_ws(d, BSGA_OP_SPECIAL_DENSE, ws, ws_bytes));
  if (d.ns == 0) return BSGA_OK;
  hipStream_t st = (hipStream_t)stream;
  uint16_t* kp = (uint16_t*)ws;
  uint16_t* vt = kp + (size_t)d.H * d.ntot_pad * kHeadDim;
  BSGA_TRY(hip_status(launch_pack(d, k, v, kp, vt, st)));
  return hip_status(launch_special(d, q, kp, vt, o, lse, (char*)ws + ws_pack(d), st));
}

int bsga_dense_attn(const bsga_shape* shape, const uint16_t* q, const uint16_t* k,
                    const uint16_t* v, uint16_t* o, float* lse, void* ws, size_t ws_bytes,
                    void* stream) {
  BSGA_TRY(check_shape(shape));
  const Dims d = make_dims(*shape);
  BSGA_TRY(check_qkv(q, k, v));
  BSGA_TRY(check_ptr(o, 16));
  BSGA_TRY(check_ptr(lse, 4));
  BSGA_TRY(check_ws(d, BSGA_OP_DENSE_ATTN, ws, ws_bytes));
  hipStream_t st = (hipStream_t)stream;
  uint16_t* kp = (uint16_t*)ws;
  uint16_t* vt = kp + (size_t)d.H * d.ntot_pad * kHeadDim;
  BSGA_TRY(hip_status(launch_pack(d, k, v, kp, vt, st)));
  return hip_status(launch_dense(d, q, kp, vt, o, lse, st));
}

int bsga_packed_kv_bytes(const bsga_shape* shape, size_t* bytes) {
  BSGA_TRY(check_shape(shape));
  if (!bytes) return BSGA_ERR_INVALID_ARG;
  *bytes = ws_pack(make_dims(*shape));
  return BSGA_OK;
}

int bsga_pack_kv(const bsga_shape* shape, const uint16_t* k, const uint16_t* v, void* kv,
                 size_t kv_bytes, void* stream) {
  BSGA_TRY(check_shape(shape));
  const Dims d = make_dims(*shape);
  BSGA_TRY(check_ptr(k, 16));
  BSGA_TRY(check_ptr(v, 16));
  BSGA_TRY(check_packed(d, kv, kv_bytes));
  uint16_t* kp = (uint16_t*)kv;
  return hip_status(launch_pack(d, k, v, kp, kp + (size_t)d.H * d.ntot_pad * kHeadDim,
                                (hipStream_t)stream));
}

int bsga_sparse_attn_packed(const bsga_shape* shape, const uint16_t* q, const void* kv,
                            size_t kv_bytes, const int32_t* row_ptr, const int32_t* col_idx,
                            uint16_t* o, float* lse, void* stream) {
  BSGA_TRY(check_shape(shape));
  const Dims d = make_dims(*shape);
  BSGA_TRY(check_ptr(q, 16));
  BSGA_TRY(check_packed(d, kv, kv_bytes));
  BSGA_TRY(check_ptr(row_ptr, 4));
  BSGA_TRY(check_ptr(col_idx, 4));
  BSGA_TRY(check_ptr(o, 16));
  BSGA_TRY(check_ptr(lse, 4));
  const uint16_t* kp = (const uint16_t*)kv;
  return hip_status(launch_sparse_attn(d, q, kp, kp + (size_t)d.H * d.ntot_pad * kHeadDim,
                                       row_ptr, col_idx, o, lse, (hipStream_t)stream));
}

int bsga_special_dense_packed(const bsga_shape* shape, const uint16_t* q, const void* kv,
                              size_t kv_bytes, uint16_t* o, float* lse, void* ws,
                              size_t ws_bytes, void* stream) {
  BSGA_TRY(check_shape(shape));
  const Dims d = make_dims(*shape);
  BSGA_TRY(check_ptr(q, 16));
  BSGA_TRY(check_packed(d, kv, kv_bytes));
  BSGA_TRY(check_ptr(o, 16));
  BSGA_TRY(check_ptr(lse, 4));
  BSGA_TRY(check_ws(d, BSGA_OP_SPECIAL_DENSE_PACKED, ws, ws_bytes));
  const uint16_t* kp = (const uint16_t*)kv;
  return hip_status(launch_special(d, q, kp, kp + (size_t)d.H * d.ntot_pad * kHeadDim, o, lse,
                                   ws, (hipStream_t)stream));
}

int bsga_dense_attn_packed(const bsga_shape* shape, const uint16_t* q, const void* kv,
                           size_t kv_bytes, uint16_t* o, float* lse, void* stream) {
  BSGA_TRY(check_shape(shape));
  const Dims d = make_dims(*shape);
  BSGA_TRY(check_ptr(q, 16));
  BSGA_TRY(check_packed(d, kv, kv_bytes));
  BSGA_TRY(check_ptr(o, 16));
  BSGA_TRY(check_ptr(lse, 4));
  const uint16_t* kp = (const uint16_t*)kv;
  return hip_status(launch_dense(d, q, kp, kp + (size_t)d.H * d.ntot_pad * kHeadDim, o, lse,
                                 (hipStream_t)stream));
}

int bsga_patch_rows_packed(const bsga_shape* shape, const uint16_t* q, const void* kv,
                           size_t kv_bytes, const int32_t* row_ptr, const int32_t* col_idx,
                           uint16_t* o, float* lse, void* ws, size_t ws_bytes, void* stream) {
  BSGA_TRY(check_shape(shape));
  const Dims d = make_dims(*shape);
  BSGA_TRY(check_ptr(q, 16));
  BSGA_TRY(check_packed(d, kv, kv_bytes));
  BSGA_TRY(check_ptr(row_ptr, 4));
  BSGA_TRY(check_ptr(col_idx, 4));
  BSGA_TRY(check_ptr(o, 16));
  BSGA_TRY(check_ptr(lse, 4));
  if (ws != nullptr) BSGA_TRY(check_ws(d, BSGA_OP_PATCH_ROWS_PACKED, ws, ws_bytes));
  const uint16_t* kp = (const uint16_t*)kv;
  return hip_status(launch_patch_rows(d, q, kp, kp + (size_t)d.H * d.ntot_pad * kHeadDim,
                                      row_ptr, col_idx, o, lse, (hipStream_t)stream, ws,
                                      ws ? ws_bytes : 0));
}

int bsga_special_rows_packed(const bsga_shape* shape, const uint16_t* q, const void* kv,
                             size_t kv_bytes, uint16_t* o, float* lse, void* ws,
                             size_t ws_bytes, void* stream) {
  BSGA_TRY(check_shape(shape));
  const Dims d = make_dims(*shape);
  BSGA_TRY(check_ptr(q, 16));
  BSGA_TRY(check_packed(d, kv, kv_bytes));
  BSGA_TRY(check_ptr(o, 16));
  BSGA_TRY(check_ptr(lse, 4));
  BSGA_TRY(check_ws(d, BSGA_OP_SPECIAL_DENSE_PACKED, ws, ws_bytes));
  const uint16_t* kp = (const uint16_t*)kv;
  return hip_status(launch_special_rows(d, q, kp, kp + (size_t)d.H * d.ntot_pad * kHeadDim, o,
                                        lse, ws, (hipStream_t)stream));
}

static int layer_impl(const bsga_shape* shape, const uint16_t* q, const uint16_t* k,
                      const uint16_t* v, const double* rho_per_head, double rho, double tau,
                      float* probs, int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                      uint16_t* o, float* lse, float* o32, bool train, void* ws,
                      size_t ws_bytes, void* stream) {
  BSGA_TRY(check_shape(shape));
  const Dims d = make_dims(*shape);
  BSGA_TRY(check_select_shape(d));
  BSGA_TRY(check_qkv(q, k, v));
  BSGA_TRY(check_ptr(probs, 4));
  BSGA_TRY(check_csr(d, row_ptr, col_idx, col_capacity));
  BSGA_TRY(check_ptr(o, 16));
  BSGA_TRY(check_ptr(lse, 4));
  if (train) {
    BSGA_TRY(check_ptr(o32, 16));
    if (!patch_rows_train_supported(d)) return BSGA_ERR_UNSUPPORTED;
  }
  SelectParams sp;
  BSGA_TRY(fill_select_params(d, rho_per_head, rho, tau, &sp));
  BSGA_TRY(check_ws(d, BSGA_OP_LAYER, ws, ws_bytes));
  hipStream_t st = (hipStream_t)stream;
  uint16_t* kp = (uint16_t*)ws;
  uint16_t* vt = kp + (size_t)d.H * d.ntot_pad * kHeadDim;
  char* scratch = (char*)ws + ws_pack(d);
  const size_t half = up((size_t)d.H * d.B * kHeadDim * sizeof(float));
  float* qb = (float*)scratch;
  float* kb = (float*)(scratch + half);
  BSGA_TRY(hip_status(launch_pool(d, q, k, qb, kb, st)));
  BSGA_TRY(hip_status(launch_scores(d, qb, kb, probs, nullptr, st)));
  BSGA_TRY(hip_status(launch_softmax(d, probs, st)));
  BSGA_TRY(hip_status(launch_select(d, probs, sp, row_ptr, col_idx, scratch, st)));
  BSGA_TRY(hip_status(launch_pack(d, k, v, kp, vt, st)));
  BSGA_TRY(hip_status(launch_patch_rows(d, q, kp, vt, row_ptr, col_idx, o, lse, st, scratch,
                                        ws_bytes - ws_pack(d), o32)));
  return hip_status(launch_special_rows(d, q, kp, vt, o, lse, scratch, st, o32));
}

int bsga_layer(const bsga_shape* shape, const uint16_t* q, const uint16_t* k, const uint16_t* v,
               const double* rho_per_head, double rho, double tau, float* probs, int32_t* row_ptr,
               int32_t* col_idx, int64_t col_capacity, uint16_t* o, float* lse, void* ws,
               size_t ws_bytes, void* stream) {
  return layer_impl(shape, q, k, v, rho_per_head, rho, tau, probs, row_ptr, col_idx, col_capacity,
                    o, lse, nullptr, false, ws, ws_bytes, stream);
}

int bsga_layer_train(const bsga_shape* shape, const uint16_t* q, const uint16_t* k,
                     const uint16_t* v, const double* rho_per_head, double rho, double tau,
                     float* probs, int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                     uint16_t* o, float* lse, float* o32, void* ws, size_t ws_bytes,
                     void* stream) {
  return layer_impl(shape, q, k, v, rho_per_head, rho, tau, probs, row_ptr, col_idx, col_capacity,
                    o, lse, o32, true, ws, ws_bytes, stream);
}

}  // extern "C"
