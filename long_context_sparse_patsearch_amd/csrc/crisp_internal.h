// Host-side launchers shared between the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace crisp {

struct Dims {
  int batch, n, h_q, h_kv, d;
  int nb;          // key/query blocks per sequence
  int group;       // h_q / h_kv
  int64_t bh;      // batch * h_q
  int64_t rows;    // batch * h_q * nb (CSR rows)
  int64_t tri;     // nb * (nb + 1) / 2 (causal cells per head)
};

// ---- routing (route.hip) ----
// Split of the key range into chunks for the proxy passes.
int proxy_chunk_tiles(const Dims& dm);
int proxy_num_chunks(const Dims& dm);
struct RouteBufs {
  float* part;    // [bh][chunks][128][2]  per row and chunk: maximum, normaliser
  float* stats;   // [bh][128][2]          per row: maximum, 1 / normaliser
  float* tile;    // [bh][nb][3][128]      per tile and row: maximum, lower and upper sums
  float* lu;      // [bh][nb][2]           per key block: L, U
};
hipError_t launch_route(const Dims& dm, float tau, const uint16_t* q, const uint16_t* k,
                        float* c_struct, int8_t* pattern, float* p_vert, float* p_slash,
                        const RouteBufs& ws, hipStream_t st);
// Device address of the current GPU's static routing scratch (CRISP_ROUTE_SCRATCH_BYTES).
hipError_t route_scratch(void** ptr);

// ---- selection (select.hip) ----
struct SelectWs {
  uint8_t* vsflags;     // [bh][2][nb]
  float* qbar;          // [bh][nb][d]
  float* kbar;          // [batch*h_kv][nb][d]
  float* abar;          // [bh][tri]  scaled logits, then x = A_bar / nb
  unsigned long long* hist_mass;  // [bh][2048]
  unsigned long long* pe_state;   // [bh][8]
  int64_t* rowcnt;      // [rows]
  int32_t* eqcnt;       // [rows]
  int32_t* seltake;     // [rows]
  int64_t* scan_part;   // [scan blocks + 1]
  unsigned long long* pe_rowst;   // [rows][2] per-row cut of the per-row PE variant: key T, cells equal to T taken
};
size_t select_ws_layout(const Dims& dm, SelectWs* ws, char* base);
// vs_rule: VS_NOISE_FLOOR (CRISP's VSIndex), VS_GAMMA_CUMSUM (FlexPrefill's budget rule) or
// VS_MEDIAN_FLOOR (the noise floor with the median of the non-anchor scores); band: a selected
// slash block also selects block diagonal delta + 1.
enum { VS_NOISE_FLOOR = 0, VS_GAMMA_CUMSUM = 1, VS_MEDIAN_FLOOR = 2 };
hipError_t launch_select(const Dims& dm, float alpha, float gamma, int kmin_blocks,
                         const uint16_t* q, const uint16_t* k, const int8_t* pattern,
                         const float* p_vert, const float* p_slash, int64_t* row_ptr,
                         int32_t* col_idx, uint8_t* sel_mask, const SelectWs& ws, hipStream_t st,
                         int vs_rule = VS_NOISE_FLOOR, int band = 0, int pe_rows = 0);

// ---- measurement (probe.hip) ----
constexpr int PROBE_SINK_FLOATS = 4096;
// flop: the launch's work (host); operands: 65536 bytes of bf16 pairs (device)
hipError_t launch_mfma_probe(const void* operands, float* sink, int iters, double* flop, hipStream_t st);

// ---- the FlexPrefill baseline path (flex.hip) ----
// ws: flex_route_ws_bytes(dm) bytes (pooled keys of every KV group)
size_t flex_route_ws_bytes(const Dims& dm);
hipError_t launch_flex_route(const Dims& dm, float tau, const uint16_t* q, const uint16_t* k, const float* p_vert,
                             float* jsd, int8_t* pattern, float* kbar, hipStream_t st);
hipError_t launch_flex_vs(const Dims& dm, float gamma, int kmin_blocks, const int8_t* pattern, const float* p_vert,
                          const float* p_slash, uint8_t* vsflags, uint8_t* sel_mask, hipStream_t st);
hipError_t launch_median_vs(const Dims& dm, float alpha, int kmin_blocks, const int8_t* pattern, const float* p_vert,
                            const float* p_slash, uint8_t* vsflags, uint8_t* sel_mask, hipStream_t st);

// ---- attention (attn.hip) ----
// ws: attn_ws_bytes(dm) bytes of scratch (work-queue counters and a V^T copy)
size_t attn_ws_bytes(const Dims& dm);
hipError_t launch_sparse_attn(const Dims& dm, const uint16_t* q, const uint16_t* k,
                              const uint16_t* v, const int64_t* row_ptr, const int32_t* col_idx,
                              int64_t col_capacity, void* out, int out_bf16, void* ws, hipStream_t st);
hipError_t launch_dense_attn(const Dims& dm, const uint16_t* q, const uint16_t* k,
                             const uint16_t* v, void* out, int out_bf16, void* ws, hipStream_t st);

}  // namespace crisp
