// C-ABI entry points of libcrisp: argument validation (host only, before any
// HIP call), workspace carving and launch sequencing on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>

#include "../../include/crisp.h"
#include "crisp_internal.h"

using crisp::Dims;

namespace {

thread_local char g_err[256] = "";

constexpr int kBlock = 128;
constexpr int kMinN = 3 * kBlock;
constexpr int kMaxN = 1 << 20;

int make_dims(const crisp_shape* s, Dims* dm) {
  if (!s) return CRISP_ERR_NULL;
  if (s->batch < 0 || s->h_q < 1 || s->h_kv < 1 || s->h_q % s->h_kv) return CRISP_ERR_SHAPE;
  if (s->d != 64 && s->d != 128) return CRISP_ERR_SHAPE;
  if (s->n % kBlock || s->n < kMinN || s->n > kMaxN) return CRISP_ERR_SHAPE;
  const int64_t bh = (int64_t)s->batch * s->h_q;
  const int64_t nb = s->n / kBlock;
  // grid limits: batch*h_q is a grid dimension; one workgroup of up to 256 threads per CSR row
  if (bh > 65535 || bh * nb > (1LL << 24) - 1) return CRISP_ERR_SHAPE;
  dm->batch = s->batch;
  dm->n = s->n;
  dm->h_q = s->h_q;
  dm->h_kv = s->h_kv;
  dm->d = s->d;
  dm->nb = (int)nb;
  dm->group = s->h_q / s->h_kv;
  dm->bh = bh;
  dm->rows = bh * nb;
  dm->tri = nb * (nb + 1) / 2;
  return CRISP_OK;
}

int check_cfg(const crisp_cfg* c) {
  if (!c) return CRISP_ERR_NULL;
  if (c->block != kBlock || c->last_q != kBlock || c->w_sink != kBlock || c->w_local != kBlock)
    return CRISP_ERR_UNSUPPORTED;
  if (c->k_min_tokens < 0 || c->k_min_tokens % kBlock) return CRISP_ERR_PARAM;
  if (!std::isfinite(c->tau)) return CRISP_ERR_PARAM;
  if (!std::isfinite(c->alpha) || !(c->alpha >= 0.f)) return CRISP_ERR_PARAM;
  if (!(c->gamma > 0.f && c->gamma <= 1.f)) return CRISP_ERR_PARAM;
  return CRISP_OK;
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

using RouteWs = crisp::RouteBufs;

size_t route_ws_layout(const Dims& dm, RouteWs* w, char* base) {
  const int nch = crisp::proxy_num_chunks(dm);
  size_t off = 0;
  auto take = [&](size_t bytes) -> char* {
    char* p = base ? base + off : nullptr;
    off += align256(bytes);
    return p;
  };
  RouteWs r{};
  r.part = (float*)take((size_t)dm.bh * nch * kBlock * 2 * sizeof(float));
  r.stats = (float*)take((size_t)dm.bh * kBlock * 2 * sizeof(float));
  r.tile = (float*)take((size_t)dm.bh * dm.nb * 3 * kBlock * sizeof(float));
  r.lu = (float*)take((size_t)dm.bh * dm.nb * 2 * sizeof(float));
  if (w) *w = r;
  return off;
}

size_t ws_bytes_for(const Dims& dm, int call) {
  switch (call) {
    case CRISP_CALL_ROUTE: return route_ws_layout(dm, nullptr, nullptr);
    case CRISP_CALL_SELECT: return crisp::select_ws_layout(dm, nullptr, nullptr);
    case CRISP_CALL_ATTN: return crisp::attn_ws_bytes(dm);
    case CRISP_CALL_DENSE: return crisp::attn_ws_bytes(dm);
    case CRISP_CALL_FLEX_ROUTE: return crisp::flex_route_ws_bytes(dm);
    case CRISP_CALL_FLEX_SELECT: return crisp::select_ws_layout(dm, nullptr, nullptr);
    default: return (size_t)-1;
  }
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return CRISP_OK;
  std::snprintf(g_err, sizeof(g_err), "%s: %s", hipGetErrorName(e), hipGetErrorString(e));
  return CRISP_ERR_HIP;
}

}  // namespace

extern "C" {

int crisp_workspace_bytes(const crisp_shape* shape, const crisp_cfg* cfg, int call, size_t* bytes) {
  Dims dm;
  int st = make_dims(shape, &dm);
  if (st) return st;
  if ((st = check_cfg(cfg))) return st;
  if (!bytes) return CRISP_ERR_NULL;
  const size_t b = ws_bytes_for(dm, call);
  if (b == (size_t)-1) return CRISP_ERR_PARAM;
  *bytes = dm.batch ? b : 0;
  return CRISP_OK;
}

int crisp_max_blocks(const crisp_shape* shape, int64_t* blocks) {
  Dims dm;
  const int st = make_dims(shape, &dm);
  if (st) return st;
  if (!blocks) return CRISP_ERR_NULL;
  *blocks = dm.bh * dm.tri;
  return CRISP_OK;
}

int crisp_use_dense(const crisp_shape* shape, int32_t* use_dense) {
  Dims dm;
  const int st = make_dims(shape, &dm);
  if (st) return st;
  if (!use_dense) return CRISP_ERR_NULL;
  *use_dense = dm.n < CRISP_DENSE_BELOW_TOKENS ? 1 : 0;
  return CRISP_OK;
}

int crisp_route(const crisp_shape* shape, const crisp_cfg* cfg, const void* q_bf16, const void* k_bf16,
                float* c_struct, int8_t* pattern, float* p_vert, float* p_slash, void* ws, size_t ws_bytes,
                void* stream) {
  Dims dm;
  int st = make_dims(shape, &dm);
  if (st) return st;
  if ((st = check_cfg(cfg))) return st;
  if (dm.batch == 0) return CRISP_OK;
  if (!q_bf16 || !k_bf16 || !c_struct || !pattern || !p_vert || !p_slash || !ws) return CRISP_ERR_NULL;
  if (misaligned(q_bf16) || misaligned(k_bf16) || misaligned(c_struct) || misaligned(pattern) ||
      misaligned(p_vert) || misaligned(p_slash) || misaligned(ws))
    return CRISP_ERR_ALIGN;
  RouteWs w;
  if (ws_bytes < route_ws_layout(dm, &w, static_cast<char*>(ws))) return CRISP_ERR_WORKSPACE;
  return hip_status(crisp::launch_route(dm, cfg->tau, static_cast<const uint16_t*>(q_bf16),
                                        static_cast<const uint16_t*>(k_bf16), c_struct, pattern, p_vert, p_slash,
                                        w, static_cast<hipStream_t>(stream)));
}

int crisp_route_noalloc(const crisp_shape* shape, const crisp_cfg* cfg, const void* q_bf16, const void* k_bf16,
                        float* c_struct, int8_t* pattern, float* p_vert, float* p_slash, void* stream) {
  Dims dm;
  int st = make_dims(shape, &dm);
  if (st) return st;
  if ((st = check_cfg(cfg))) return st;
  if (dm.batch == 0) return CRISP_OK;
  if (!q_bf16 || !k_bf16 || !c_struct || !pattern || !p_vert || !p_slash) return CRISP_ERR_NULL;
  if (misaligned(q_bf16) || misaligned(k_bf16) || misaligned(c_struct) || misaligned(pattern) ||
      misaligned(p_vert) || misaligned(p_slash))
    return CRISP_ERR_ALIGN;
  if (route_ws_layout(dm, nullptr, nullptr) > (size_t)CRISP_ROUTE_SCRATCH_BYTES) return CRISP_ERR_SCRATCH;
  void* ws = nullptr;
  if ((st = hip_status(crisp::route_scratch(&ws)))) return st;
  RouteWs w;
  route_ws_layout(dm, &w, static_cast<char*>(ws));
  return hip_status(crisp::launch_route(dm, cfg->tau, static_cast<const uint16_t*>(q_bf16),
                                        static_cast<const uint16_t*>(k_bf16), c_struct, pattern, p_vert, p_slash,
                                        w, static_cast<hipStream_t>(stream)));
}

static int select_common(const crisp_shape* shape, const crisp_cfg* cfg, const void* q_bf16, const void* k_bf16,
                         const int8_t* pattern, const float* p_vert, const float* p_slash, int64_t* row_ptr,
                         int32_t* col_idx, int64_t col_capacity, uint8_t* sel_mask, void* ws, size_t ws_bytes,
                         void* stream, int vs_rule, int band, int pe_rows = 0) {
  Dims dm;
  int st = make_dims(shape, &dm);
  if (st) return st;
  if ((st = check_cfg(cfg))) return st;
  if (dm.batch == 0) return CRISP_OK;
  if (!q_bf16 || !k_bf16 || !pattern || !p_vert || !p_slash || !row_ptr || !col_idx || !ws) return CRISP_ERR_NULL;
  if (misaligned(q_bf16) || misaligned(k_bf16) || misaligned(pattern) || misaligned(p_vert) ||
      misaligned(p_slash) || misaligned(row_ptr) || misaligned(col_idx) || misaligned(ws) ||
      (sel_mask && misaligned(sel_mask)))
    return CRISP_ERR_ALIGN;
  crisp::SelectWs w;
  if (ws_bytes < crisp::select_ws_layout(dm, &w, static_cast<char*>(ws))) return CRISP_ERR_WORKSPACE;
  if (col_capacity < dm.bh * dm.tri) return CRISP_ERR_CAPACITY;
  return hip_status(crisp::launch_select(dm, cfg->alpha, cfg->gamma, cfg->k_min_tokens / kBlock,
                                         static_cast<const uint16_t*>(q_bf16), static_cast<const uint16_t*>(k_bf16),
                                         pattern, p_vert, p_slash, row_ptr, col_idx, sel_mask, w,
                                         static_cast<hipStream_t>(stream), vs_rule, band, pe_rows));
}

int crisp_select(const crisp_shape* shape, const crisp_cfg* cfg, const void* q_bf16, const void* k_bf16,
                 const int8_t* pattern, const float* p_vert, const float* p_slash, int64_t* row_ptr,
                 int32_t* col_idx, int64_t col_capacity, uint8_t* sel_mask, void* ws, size_t ws_bytes,
                 void* stream) {
  return select_common(shape, cfg, q_bf16, k_bf16, pattern, p_vert, p_slash, row_ptr, col_idx, col_capacity,
                       sel_mask, ws, ws_bytes, stream, crisp::VS_NOISE_FLOOR, 0);
}

int crisp_select_variant(const crisp_shape* shape, const crisp_cfg* cfg, int variant, const void* q_bf16,
                         const void* k_bf16, const int8_t* pattern, const float* p_vert, const float* p_slash,
                         int64_t* row_ptr, int32_t* col_idx, int64_t col_capacity, uint8_t* sel_mask, void* ws,
                         size_t ws_bytes, void* stream) {
  if (variant & ~(CRISP_VARIANT_MEDIAN_FLOOR | CRISP_VARIANT_SLASH_BAND | CRISP_VARIANT_PE_PER_ROW))
    return CRISP_ERR_PARAM;
  const int rule = (variant & CRISP_VARIANT_MEDIAN_FLOOR) ? crisp::VS_MEDIAN_FLOOR : crisp::VS_NOISE_FLOOR;
  return select_common(shape, cfg, q_bf16, k_bf16, pattern, p_vert, p_slash, row_ptr, col_idx, col_capacity,
                       sel_mask, ws, ws_bytes, stream, rule, (variant & CRISP_VARIANT_SLASH_BAND) ? 1 : 0,
                       (variant & CRISP_VARIANT_PE_PER_ROW) ? 1 : 0);
}

int flex_select(const crisp_shape* shape, const crisp_cfg* cfg, const void* q_bf16, const void* k_bf16,
                const int8_t* pattern, const float* p_vert, const float* p_slash, int64_t* row_ptr,
                int32_t* col_idx, int64_t col_capacity, uint8_t* sel_mask, void* ws, size_t ws_bytes,
                void* stream) {
  return select_common(shape, cfg, q_bf16, k_bf16, pattern, p_vert, p_slash, row_ptr, col_idx, col_capacity,
                       sel_mask, ws, ws_bytes, stream, crisp::VS_GAMMA_CUMSUM, 0);
}

int flex_route(const crisp_shape* shape, const crisp_cfg* cfg, float tau_jsd, const void* q_bf16,
               const void* k_bf16, const float* p_vert, float* jsd, int8_t* pattern, void* ws, size_t ws_bytes,
               void* stream) {
  Dims dm;
  int st = make_dims(shape, &dm);
  if (st) return st;
  if ((st = check_cfg(cfg))) return st;
  if (!(tau_jsd >= 0.f) || !std::isfinite(tau_jsd)) return CRISP_ERR_PARAM;
  if (dm.batch == 0) return CRISP_OK;
  if (!q_bf16 || !k_bf16 || !p_vert || !jsd || !pattern || !ws) return CRISP_ERR_NULL;
  if (misaligned(q_bf16) || misaligned(k_bf16) || misaligned(p_vert) || misaligned(jsd) || misaligned(pattern) ||
      misaligned(ws))
    return CRISP_ERR_ALIGN;
  if (ws_bytes < crisp::flex_route_ws_bytes(dm)) return CRISP_ERR_WORKSPACE;
  return hip_status(crisp::launch_flex_route(dm, tau_jsd, static_cast<const uint16_t*>(q_bf16),
                                             static_cast<const uint16_t*>(k_bf16), p_vert, jsd, pattern,
                                             static_cast<float*>(ws), static_cast<hipStream_t>(stream)));
}

int crisp_sparse_attn(const crisp_shape* shape, const crisp_cfg* cfg, const void* q_bf16, const void* k_bf16,
                      const void* v_bf16, const int64_t* row_ptr, const int32_t* col_idx, int64_t col_capacity,
                      void* out, int out_dtype, void* ws, size_t ws_bytes, void* stream) {
  Dims dm;
  int st = make_dims(shape, &dm);
  if (st) return st;
  if ((st = check_cfg(cfg))) return st;
  if (out_dtype != CRISP_OUT_F32 && out_dtype != CRISP_OUT_BF16) return CRISP_ERR_PARAM;
  if (col_capacity < 0) return CRISP_ERR_PARAM;
  if (dm.batch == 0) return CRISP_OK;
  if (!q_bf16 || !k_bf16 || !v_bf16 || !row_ptr || !out) return CRISP_ERR_NULL;
  if (col_capacity > 0 && !col_idx) return CRISP_ERR_NULL;
  if (!ws) return CRISP_ERR_NULL;
  if (misaligned(q_bf16) || misaligned(k_bf16) || misaligned(v_bf16) || misaligned(row_ptr) ||
      (col_idx && misaligned(col_idx)) || misaligned(out) || misaligned(ws))
    return CRISP_ERR_ALIGN;
  if (ws_bytes < ws_bytes_for(dm, CRISP_CALL_ATTN)) return CRISP_ERR_WORKSPACE;
  return hip_status(crisp::launch_sparse_attn(dm, static_cast<const uint16_t*>(q_bf16),
                                              static_cast<const uint16_t*>(k_bf16),
                                              static_cast<const uint16_t*>(v_bf16), row_ptr, col_idx, col_capacity,
                                              out, out_dtype == CRISP_OUT_BF16, ws, static_cast<hipStream_t>(stream)));
}

int dense_attn(const crisp_shape* shape, const void* q_bf16, const void* k_bf16, const void* v_bf16, void* out,
               int out_dtype, void* ws, size_t ws_bytes, void* stream) {
  Dims dm;
  const int st = make_dims(shape, &dm);
  if (st) return st;
  if (out_dtype != CRISP_OUT_F32 && out_dtype != CRISP_OUT_BF16) return CRISP_ERR_PARAM;
  if (dm.batch == 0) return CRISP_OK;
  if (!q_bf16 || !k_bf16 || !v_bf16 || !out || !ws) return CRISP_ERR_NULL;
  if (misaligned(q_bf16) || misaligned(k_bf16) || misaligned(v_bf16) || misaligned(out) || misaligned(ws))
    return CRISP_ERR_ALIGN;
  if (ws_bytes < ws_bytes_for(dm, CRISP_CALL_DENSE)) return CRISP_ERR_WORKSPACE;
  return hip_status(crisp::launch_dense_attn(dm, static_cast<const uint16_t*>(q_bf16),
                                             static_cast<const uint16_t*>(k_bf16),
                                             static_cast<const uint16_t*>(v_bf16), out,
                                             out_dtype == CRISP_OUT_BF16, ws, static_cast<hipStream_t>(stream)));
}

int crisp_mfma_probe(const void* operands, float* sink, int iters, double* flop, void* stream) {
  if (!operands || !sink || !flop) return CRISP_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(operands) % 16 || reinterpret_cast<uintptr_t>(sink) % 4) return CRISP_ERR_ALIGN;
  if (iters < 1 || iters > 10000000) return CRISP_ERR_PARAM;
  static_assert(crisp::PROBE_SINK_FLOATS == CRISP_PROBE_SINK_FLOATS, "sink size");
  return hip_status(crisp::launch_mfma_probe(operands, sink, iters, flop, static_cast<hipStream_t>(stream)));
}

const char* crisp_status_string(int status) {
  switch (status) {
    case CRISP_OK: return "ok";
    case CRISP_ERR_NULL: return "a required pointer is NULL";
    case CRISP_ERR_SHAPE: return "shape outside the supported range";
    case CRISP_ERR_PARAM: return "setting out of range";
    case CRISP_ERR_UNSUPPORTED: return "setting not supported by this implementation";
    case CRISP_ERR_WORKSPACE: return "workspace smaller than crisp_workspace_bytes";
    case CRISP_ERR_CAPACITY: return "col_capacity below crisp_max_blocks";
    case CRISP_ERR_HIP: return "HIP launch failed";
    case CRISP_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case CRISP_ERR_SCRATCH: return "shape needs more scratch than the static routing buffer holds";
    default: return "unknown status";
  }
}

const char* crisp_last_error(void) { return g_err; }

}  // extern "C"
