// C ABI of libnabla (declared in include/nabla.h): argument validation,
// geometry derivation and kernel launches.  Every check runs before anything
// is enqueued; no entry point allocates memory, synchronizes or throws.
#include <math.h>
#include <string.h>

#include <atomic>

#include "../../include/nabla.h"
#include "nabla_common.hpp"

using nabla::Geo;

namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return NABLA_OK;
  g_last_hip_error = (int)e;
  return NABLA_E_HIP;
}

// Validate the geometry and derive the kernels' view of it.  `layout_used`
// is false for entry points whose tensor layout is fixed by the call.
int make_geo(const nabla_geom* p, bool layout_used, Geo* g, bool* empty) {
  if (p == nullptr) return NABLA_E_NULL;
  if (p->batch < 0 || p->heads < 0) return NABLA_E_SHAPE;
  if (p->T < 1 || p->H < 1 || p->W < 1) return NABLA_E_SHAPE;
  if (p->P != nabla::kP) return NABLA_E_PATCH;
  if (p->head_dim != 64 && p->head_dim != 128) return NABLA_E_HEAD_DIM;
  if (p->dtype != NABLA_DTYPE_F32 && p->dtype != NABLA_DTYPE_BF16) return NABLA_E_DTYPE;
  if (p->out_dtype != NABLA_DTYPE_F32 && p->out_dtype != NABLA_DTYPE_BF16) return NABLA_E_DTYPE;
  if (p->dtype == NABLA_DTYPE_F32 && p->out_dtype != NABLA_DTYPE_F32) return NABLA_E_DTYPE;
  if (layout_used && p->layout != NABLA_LAYOUT_THW && p->layout != NABLA_LAYOUT_BLOCKED)
    return NABLA_E_LAYOUT;
  const int64_t gh = (p->H + 7) / 8, gw = (p->W + 7) / 8;
  if (p->H > (1 << 20) || p->W > (1 << 20) || p->T > (1 << 20)) return NABLA_E_SHAPE;
  const int64_t nb = (int64_t)p->T * gh * gw;
  if (nb > NABLA_MAX_BLOCKS) return NABLA_E_TOO_LARGE;
  const int64_t bh = p->batch * p->heads;
  if (p->batch != 0 && bh / p->batch != p->heads) return NABLA_E_SHAPE;
  if (bh > 65535) return NABLA_E_SHAPE;             // one grid row per head in the mask kernels
  const int64_t thw = (int64_t)p->T * p->H * p->W * p->head_dim;
  const int64_t blk = nb * nabla::kN * p->head_dim;
  if (thw >= (int64_t)1 << 31 || blk >= (int64_t)1 << 31) return NABLA_E_SHAPE;
  g->bh = bh;
  g->T = p->T;
  g->H = p->H;
  g->W = p->W;
  g->gh = (int)gh;
  g->gw = (int)gw;
  g->nb = (int)nb;
  g->d = p->head_dim;
  g->layout = p->layout == NABLA_LAYOUT_BLOCKED ? 1 : 0;
  g->head_elems = (int)(g->layout == 1 ? blk : thw);
  g->per_frame_r = nabla::make_recip((uint32_t)(gh * gw));
  g->gw_r = nabla::make_recip((uint32_t)gw);
  *empty = bh == 0;
  return NABLA_OK;
}

int check_sta(const int32_t* sta, int out[3]) {
  out[0] = out[1] = out[2] = 0;
  if (sta == nullptr) return NABLA_OK;
  const bool all_zero = sta[0] == 0 && sta[1] == 0 && sta[2] == 0;
  if (all_zero) return NABLA_OK;
  for (int i = 0; i < 3; ++i) {
    if (sta[i] <= 0 || (sta[i] & 1) == 0) return NABLA_E_STA;
    out[i] = sta[i];
  }
  return NABLA_OK;
}

// thr in (0, 1]; 0 (adaptive part off, pure STA) only with an STA window
bool thr_ok(float thr, const int win[3]) {
  if (!isfinite(thr) || thr < 0.0f || thr > 1.0f) return false;
  return thr > 0.0f || win[0] > 0;
}
bool scale_ok(float s) { return isfinite(s) && s > 0.0f; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr int kWsParts = 7;

void workspace_parts(const Geo& g, bool bf16, size_t off[kWsParts], size_t* total) {
  const size_t bh = (size_t)g.bh, nb = (size_t)g.nb, nw = (nb + 31) / 32;
  const size_t sizes[kWsParts] = {
      bh * nb * g.d * sizeof(float),        // qbar
      bh * (size_t)nabla::kbar_head_elems(g.nb, g.d) * 2,   // kbar (split parts, tiled)
      bh * nb * nw * sizeof(uint32_t),      // mask bits
      bh * nb * sizeof(int32_t),            // row counts
      bh * (nb + 1) * sizeof(int32_t),      // row_ptr
      bh * nb * nb * sizeof(int32_t),       // col_idx
      bf16 ? bh * nb * 64 * g.d * 2 : 0,    // V^T
  };
  size_t at = 0;
  for (int i = 0; i < kWsParts; ++i) {
    off[i] = at;
    at = align256(at + sizes[i]);
  }
  *total = at;
}

hipStream_t as_stream(void* s) { return (hipStream_t)s; }

// Checks shared by the two whole-call entry points, in the order nabla_forward
// documents; NABLA_OK with g->bh == 0 means nothing to do.
int check_forward(const nabla_geom* geom, const void* q, const void* k, const void* v, float thr,
                  const int32_t* sta, float scale, const void* o, Geo* g, int win[3]) {
  bool empty;
  int st = make_geo(geom, true, g, &empty);
  if (st != NABLA_OK) return st;
  if (!scale_ok(scale)) return NABLA_E_SCALE;
  st = check_sta(sta, win);
  if (st != NABLA_OK) return st;
  if (!thr_ok(thr, win)) return NABLA_E_THR;
  if (empty) return NABLA_OK;
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return NABLA_E_NULL;
  return NABLA_OK;
}

// One pass of the whole call over the heads of g, with its workspace parts at
// ws + off[i]: mask construction, then the attention (bf16: through V^T).
hipError_t forward_pass(const Geo& g, bool bf16, bool out_bf16, const void* q, const void* k,
                        const void* v, float thr, const int win[3], float scale, void* o,
                        char* ws, const size_t off[kWsParts], hipStream_t s) {
  float* qbar = (float*)(ws + off[0]);
  __bf16* kbar = (__bf16*)(ws + off[1]);
  uint32_t* bits = (uint32_t*)(ws + off[2]);
  int32_t* cnt = (int32_t*)(ws + off[3]);
  int32_t* rp = (int32_t*)(ws + off[4]);
  int32_t* ci = (int32_t*)(ws + off[5]);
  hipError_t e = nabla::launch_mask_build(g, bf16, q, k, qbar, kbar, thr, win, bits, cnt, nullptr,
                                          rp, ci, s);
  if (bf16) {
    void* vt = ws + off[6];
    if (e == hipSuccess) e = nabla::launch_transpose_v(g, v, vt, s);
    if (e == hipSuccess)
      e = nabla::launch_attn_fwd_vt(g, out_bf16, q, k, vt, rp, ci, scale, o, nullptr, s);
  } else if (e == hipSuccess) {
    e = nabla::launch_attn_fwd(g, false, false, q, k, v, rp, ci, scale, o, nullptr, s);
  }
  return e;
}

// Device address of this GPU's copy of `scratch` (defined below), looked up
// once per device with that device current and kept per device.
constexpr int kMaxDevices = 64;
std::atomic<char*> g_scratch_ptr[kMaxDevices];

int scratch_of_current_device(char** out);

int attn_fwd_impl(const nabla_geom* geom, const void* q, const void* k, const void* v,
                  const int32_t* row_ptr, const int32_t* col_idx, float scale, void* o,
                  float* lse, bool need_lse, void* stream) {
  Geo g;
  bool empty;
  const int st = make_geo(geom, true, &g, &empty);
  if (st != NABLA_OK) return st;
  if (!scale_ok(scale)) return NABLA_E_SCALE;
  if (empty) return NABLA_OK;
  if (q == nullptr || k == nullptr || v == nullptr || row_ptr == nullptr || col_idx == nullptr ||
      o == nullptr || (need_lse && lse == nullptr))
    return NABLA_E_NULL;
  return hip_status(nabla::launch_attn_fwd(g, geom->dtype == NABLA_DTYPE_BF16,
                                           geom->out_dtype == NABLA_DTYPE_BF16, q, k, v, row_ptr,
                                           col_idx, scale, o, lse, as_stream(stream)));
}

int attn_fwd_vt_impl(const nabla_geom* geom, const void* q, const void* k, const void* vt,
                     const int32_t* row_ptr, const int32_t* col_idx, float scale, void* o,
                     float* lse, bool need_lse, void* stream) {
  Geo g;
  bool empty;
  const int st = make_geo(geom, true, &g, &empty);
  if (st != NABLA_OK) return st;
  if (geom->dtype != NABLA_DTYPE_BF16) return NABLA_E_DTYPE;
  if (!scale_ok(scale)) return NABLA_E_SCALE;
  if (empty) return NABLA_OK;
  if (q == nullptr || k == nullptr || vt == nullptr || row_ptr == nullptr ||
      col_idx == nullptr || o == nullptr || (need_lse && lse == nullptr))
    return NABLA_E_NULL;
  return hip_status(nabla::launch_attn_fwd_vt(g, geom->out_dtype == NABLA_DTYPE_BF16, q, k, vt,
                                              row_ptr, col_idx, scale, o, lse, as_stream(stream)));
}

}  // namespace

// Workspace of nabla_forward_noalloc: a file-scope device array, one copy on
// every GPU the library runs on, held until the process ends.  On the host
// the name `scratch` stands for a host-side shadow, not device memory, so
// host code never passes it to a kernel or a copy: it uses the address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[NABLA_NOALLOC_SCRATCH_BYTES];

namespace {

int scratch_of_current_device(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return hip_status(hipErrorInvalidDevice);
  char* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    void* addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (addr == nullptr) return hip_status(hipErrorInvalidSymbol);
    p = (char*)addr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return NABLA_OK;
}

}  // namespace

extern "C" {

int nabla_abi_version(void) { return NABLA_ABI_VERSION; }

int nabla_last_hip_error(void) { return g_last_hip_error; }

const char* nabla_status_string(int status) {
  switch (status) {
    case NABLA_OK: return "ok";
    case NABLA_E_NULL: return "a required pointer is NULL";
    case NABLA_E_SHAPE: return "invalid shape (batch/heads < 0, T/H/W < 1, or sizes beyond the limits)";
    case NABLA_E_DTYPE: return "dtype/out_dtype must be F32 or BF16 (F32 inputs need F32 output)";
    case NABLA_E_HEAD_DIM: return "head_dim must be 64 or 128";
    case NABLA_E_PATCH: return "patch side P must be 8";
    case NABLA_E_THR: return "thr must be finite and in (0, 1], or 0 with an STA window";
    case NABLA_E_STA: return "STA window must be {0,0,0} or three positive odd sizes";
    case NABLA_E_WORKSPACE: return "workspace smaller than nabla_forward_workspace_size";
    case NABLA_E_LAYOUT: return "layout must be NABLA_LAYOUT_THW or NABLA_LAYOUT_BLOCKED";
    case NABLA_E_HIP: return "HIP launch failed (see nabla_last_hip_error)";
    case NABLA_E_SCALE: return "softmax scale must be finite and > 0";
    case NABLA_E_TOO_LARGE: return "more blocks per head than NABLA_MAX_BLOCKS";
    default: return "unknown status";
  }
}

int nabla_num_blocks(const nabla_geom* geom, int64_t* nb) {
  Geo g;
  bool empty;
  const int st = make_geo(geom, false, &g, &empty);
  if (st != NABLA_OK) return st;
  if (nb == nullptr) return NABLA_E_NULL;
  *nb = g.nb;
  return NABLA_OK;
}

int nabla_flatten(const nabla_geom* geom, const void* x, void* x_blocked, void* stream) {
  Geo g;
  bool empty;
  const int st = make_geo(geom, false, &g, &empty);
  if (st != NABLA_OK) return st;
  if (empty) return NABLA_OK;
  if (x == nullptr || x_blocked == nullptr) return NABLA_E_NULL;
  const int eb = geom->dtype == NABLA_DTYPE_BF16 ? 2 : 4;
  return hip_status(nabla::launch_flatten(g, eb, x, x_blocked, false, as_stream(stream)));
}

int nabla_unflatten(const nabla_geom* geom, const void* x_blocked, void* x, void* stream) {
  Geo g;
  bool empty;
  const int st = make_geo(geom, false, &g, &empty);
  if (st != NABLA_OK) return st;
  if (empty) return NABLA_OK;
  if (x == nullptr || x_blocked == nullptr) return NABLA_E_NULL;
  const int eb = geom->dtype == NABLA_DTYPE_BF16 ? 2 : 4;
  return hip_status(nabla::launch_flatten(g, eb, x_blocked, x, true, as_stream(stream)));
}

int nabla_pool(const nabla_geom* geom, const void* q, const void* k, float* qbar, void* kbar,
               void* stream) {
  Geo g;
  bool empty;
  const int st = make_geo(geom, true, &g, &empty);
  if (st != NABLA_OK) return st;
  if (empty) return NABLA_OK;
  if (q == nullptr || k == nullptr || qbar == nullptr || kbar == nullptr) return NABLA_E_NULL;
  return hip_status(nabla::launch_pool(g, geom->dtype == NABLA_DTYPE_BF16, q, k, qbar,
                                       (__bf16*)kbar, as_stream(stream)));
}

int nabla_mask(const nabla_geom* geom, const float* qbar, const void* kbar, float thr,
               const int32_t* sta, uint32_t* mask_bits, int32_t* row_count,
               uint32_t* adaptive_bits, void* stream) {
  Geo g;
  bool empty;
  int st = make_geo(geom, false, &g, &empty);
  if (st != NABLA_OK) return st;
  int win[3];
  st = check_sta(sta, win);
  if (st != NABLA_OK) return st;
  if (!thr_ok(thr, win)) return NABLA_E_THR;
  if (empty) return NABLA_OK;
  if (qbar == nullptr || kbar == nullptr || mask_bits == nullptr || row_count == nullptr)
    return NABLA_E_NULL;
  return hip_status(nabla::launch_mask(g, qbar, (const __bf16*)kbar, thr, win, mask_bits,
                                       row_count, adaptive_bits, as_stream(stream)));
}

int nabla_compact(const nabla_geom* geom, const uint32_t* mask_bits, const int32_t* row_count,
                  int32_t* row_ptr, int32_t* col_idx, void* stream) {
  Geo g;
  bool empty;
  const int st = make_geo(geom, false, &g, &empty);
  if (st != NABLA_OK) return st;
  if (empty) return NABLA_OK;
  if (mask_bits == nullptr || row_count == nullptr || row_ptr == nullptr || col_idx == nullptr)
    return NABLA_E_NULL;
  return hip_status(
      nabla::launch_compact(g, mask_bits, row_count, row_ptr, col_idx, as_stream(stream)));
}

int nabla_mask_build(const nabla_geom* geom, const void* q, const void* k, float thr,
                     const int32_t* sta, float* qbar, void* kbar, uint32_t* mask_bits,
                     int32_t* row_count, uint32_t* adaptive_bits, int32_t* row_ptr,
                     int32_t* col_idx, void* stream) {
  Geo g;
  bool empty;
  int st = make_geo(geom, true, &g, &empty);
  if (st != NABLA_OK) return st;
  int win[3];
  st = check_sta(sta, win);
  if (st != NABLA_OK) return st;
  if (!thr_ok(thr, win)) return NABLA_E_THR;
  if (empty) return NABLA_OK;
  if (q == nullptr || k == nullptr || qbar == nullptr || kbar == nullptr ||
      mask_bits == nullptr || row_count == nullptr || row_ptr == nullptr || col_idx == nullptr)
    return NABLA_E_NULL;
  return hip_status(nabla::launch_mask_build(g, geom->dtype == NABLA_DTYPE_BF16, q, k, qbar,
                                             (__bf16*)kbar, thr, win, mask_bits, row_count, adaptive_bits,
                                             row_ptr, col_idx, as_stream(stream)));
}

int nabla_attn_fwd(const nabla_geom* geom, const void* q, const void* k, const void* v,
                   const int32_t* row_ptr, const int32_t* col_idx, float scale, void* o,
                   void* stream) {
  return attn_fwd_impl(geom, q, k, v, row_ptr, col_idx, scale, o, nullptr, false, stream);
}

int nabla_attn_fwd_lse(const nabla_geom* geom, const void* q, const void* k, const void* v,
                       const int32_t* row_ptr, const int32_t* col_idx, float scale, void* o,
                       float* lse, void* stream) {
  return attn_fwd_impl(geom, q, k, v, row_ptr, col_idx, scale, o, lse, true, stream);
}

int nabla_transpose_v(const nabla_geom* geom, const void* v, void* vt, void* stream) {
  Geo g;
  bool empty;
  const int st = make_geo(geom, true, &g, &empty);
  if (st != NABLA_OK) return st;
  if (geom->dtype != NABLA_DTYPE_BF16) return NABLA_E_DTYPE;
  if (empty) return NABLA_OK;
  if (v == nullptr || vt == nullptr) return NABLA_E_NULL;
  return hip_status(nabla::launch_transpose_v(g, v, vt, as_stream(stream)));
}

int nabla_attn_fwd_vt(const nabla_geom* geom, const void* q, const void* k, const void* vt,
                      const int32_t* row_ptr, const int32_t* col_idx, float scale, void* o,
                      void* stream) {
  return attn_fwd_vt_impl(geom, q, k, vt, row_ptr, col_idx, scale, o, nullptr, false, stream);
}

int nabla_qkv_split(const nabla_geom* geom, const void* qkv, void* q, void* k, void* vt,
                    float* qbar, void* kbar, void* stream) {
  Geo g;
  bool empty;
  const int st = make_geo(geom, true, &g, &empty);
  if (st != NABLA_OK) return st;
  if (geom->dtype != NABLA_DTYPE_BF16) return NABLA_E_DTYPE;
  if (geom->layout != NABLA_LAYOUT_BLOCKED) return NABLA_E_LAYOUT;
  if (geom->batch > 65535) return NABLA_E_SHAPE;    // one grid plane per batch entry
  if (empty) return NABLA_OK;
  if (qkv == nullptr || q == nullptr || k == nullptr || vt == nullptr || qbar == nullptr ||
      kbar == nullptr)
    return NABLA_E_NULL;
  return hip_status(nabla::launch_qkv_split(g, (int)geom->batch, (int)geom->heads, qkv, q, k, vt,
                                            qbar, (__bf16*)kbar, as_stream(stream)));
}

int nabla_dense_attn_fwd(const nabla_geom* geom, const void* q, const void* k, const void* vt,
                         float scale, void* o, float* lse, void* stream) {
  Geo g;
  bool empty;
  const int st = make_geo(geom, true, &g, &empty);
  if (st != NABLA_OK) return st;
  if (geom->dtype != NABLA_DTYPE_BF16) return NABLA_E_DTYPE;
  if (!scale_ok(scale)) return NABLA_E_SCALE;
  if (empty) return NABLA_OK;
  if (q == nullptr || k == nullptr || vt == nullptr || o == nullptr) return NABLA_E_NULL;
  return hip_status(nabla::launch_attn_dense_vt(g, geom->out_dtype == NABLA_DTYPE_BF16, q, k, vt,
                                                scale, o, lse, as_stream(stream)));
}

int nabla_attn_fwd_vt_lse(const nabla_geom* geom, const void* q, const void* k, const void* vt,
                          const int32_t* row_ptr, const int32_t* col_idx, float scale, void* o,
                          float* lse, void* stream) {
  return attn_fwd_vt_impl(geom, q, k, vt, row_ptr, col_idx, scale, o, lse, true, stream);
}

int nabla_mask_transpose(const nabla_geom* geom, const uint32_t* mask_bits, uint32_t* mask_bits_t,
                         int32_t* row_count_t, void* stream) {
  Geo g;
  bool empty;
  const int st = make_geo(geom, false, &g, &empty);
  if (st != NABLA_OK) return st;
  if (empty) return NABLA_OK;
  if (mask_bits == nullptr || mask_bits_t == nullptr || row_count_t == nullptr)
    return NABLA_E_NULL;
  return hip_status(
      nabla::launch_mask_transpose(g, mask_bits, mask_bits_t, row_count_t, as_stream(stream)));
}

int nabla_attn_bwd_dq(const nabla_geom* geom, const void* q, const void* k, const void* v,
                      const void* o, const void* dout, const float* lse, const int32_t* row_ptr,
                      const int32_t* col_idx, float scale, void* dq, float* delta,
                      void* stream) {
  Geo g;
  bool empty;
  const int st = make_geo(geom, true, &g, &empty);
  if (st != NABLA_OK) return st;
  if (geom->out_dtype != geom->dtype) return NABLA_E_DTYPE;
  if (!scale_ok(scale)) return NABLA_E_SCALE;
  if (empty) return NABLA_OK;
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || dout == nullptr ||
      lse == nullptr || row_ptr == nullptr || col_idx == nullptr || dq == nullptr ||
      delta == nullptr)
    return NABLA_E_NULL;
  return hip_status(nabla::launch_attn_bwd_dq(g, geom->dtype == NABLA_DTYPE_BF16, q, k, v, o,
                                              dout, lse, row_ptr, col_idx, scale, dq, delta,
                                              as_stream(stream)));
}

int nabla_attn_bwd_dkdv(const nabla_geom* geom, const void* q, const void* k, const void* v,
                        const void* dout, const float* lse, const float* delta,
                        const int32_t* col_ptr, const int32_t* row_idx, float scale, void* dk,
                        void* dv, void* stream) {
  Geo g;
  bool empty;
  const int st = make_geo(geom, true, &g, &empty);
  if (st != NABLA_OK) return st;
  if (geom->out_dtype != geom->dtype) return NABLA_E_DTYPE;
  if (!scale_ok(scale)) return NABLA_E_SCALE;
  if (empty) return NABLA_OK;
  if (q == nullptr || k == nullptr || v == nullptr || dout == nullptr || lse == nullptr ||
      delta == nullptr || col_ptr == nullptr || row_idx == nullptr || dk == nullptr ||
      dv == nullptr)
    return NABLA_E_NULL;
  return hip_status(nabla::launch_attn_bwd_dkdv(g, geom->dtype == NABLA_DTYPE_BF16, q, k, v, dout,
                                                lse, delta, col_ptr, row_idx, scale, dk, dv,
                                                as_stream(stream)));
}

int nabla_forward_workspace_size(const nabla_geom* geom, size_t* bytes, size_t* offsets) {
  Geo g;
  bool empty;
  const int st = make_geo(geom, true, &g, &empty);
  if (st != NABLA_OK) return st;
  if (bytes == nullptr) return NABLA_E_NULL;
  size_t off[kWsParts], total;
  workspace_parts(g, geom->dtype == NABLA_DTYPE_BF16, off, &total);
  *bytes = total;
  if (offsets != nullptr) memcpy(offsets, off, sizeof(off));
  return NABLA_OK;
}

int nabla_forward(const nabla_geom* geom, const void* q, const void* k, const void* v, float thr,
                  const int32_t* sta, float scale, void* o, void* workspace,
                  size_t workspace_bytes, void* stream) {
  Geo g;
  int win[3];
  int st = check_forward(geom, q, k, v, thr, sta, scale, o, &g, win);
  if (st != NABLA_OK || g.bh == 0) return st;
  if (workspace == nullptr) return NABLA_E_NULL;
  const bool bf16 = geom->dtype == NABLA_DTYPE_BF16;
  size_t off[kWsParts], total;
  workspace_parts(g, bf16, off, &total);
  if (workspace_bytes < total) return NABLA_E_WORKSPACE;
  return hip_status(forward_pass(g, bf16, geom->out_dtype == NABLA_DTYPE_BF16, q, k, v, thr, win,
                                 scale, o, (char*)workspace, off, as_stream(stream)));
}

int nabla_forward_noalloc(const nabla_geom* geom, const void* q, const void* k, const void* v,
                          float thr, const int32_t* sta, float scale, void* o, void* stream) {
  Geo g;
  int win[3];
  int st = check_forward(geom, q, k, v, thr, sta, scale, o, &g, win);
  if (st != NABLA_OK || g.bh == 0) return st;
  const bool bf16 = geom->dtype == NABLA_DTYPE_BF16;
  const bool out_bf16 = geom->out_dtype == NABLA_DTYPE_BF16;
  // heads per pass: as many as the scratch holds (at least one, else reject)
  size_t off[kWsParts], total;
  Geo gc = g;
  gc.bh = 1;
  workspace_parts(gc, bf16, off, &total);
  if (total > (size_t)NABLA_NOALLOC_SCRATCH_BYTES) return NABLA_E_WORKSPACE;
  int64_t per_pass = (int64_t)((size_t)NABLA_NOALLOC_SCRATCH_BYTES / total);
  if (per_pass > g.bh) per_pass = g.bh;
  for (;;) {                         // per-part alignment can add a few bytes per pass
    gc.bh = per_pass;
    workspace_parts(gc, bf16, off, &total);
    if (total <= (size_t)NABLA_NOALLOC_SCRATCH_BYTES || per_pass == 1) break;
    --per_pass;
  }
  char* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != NABLA_OK) return st;
  const size_t in_head = (size_t)g.head_elems * (bf16 ? 2 : 4);
  const size_t out_head = (size_t)g.head_elems * (out_bf16 ? 2 : 4);
  const hipStream_t s = as_stream(stream);
  for (int64_t h0 = 0; h0 < g.bh; h0 += per_pass) {
    gc.bh = g.bh - h0 < per_pass ? g.bh - h0 : per_pass;
    workspace_parts(gc, bf16, off, &total);
    const hipError_t e = forward_pass(
        gc, bf16, out_bf16, (const char*)q + h0 * in_head, (const char*)k + h0 * in_head,
        (const char*)v + h0 * in_head, thr, win, scale, (char*)o + h0 * out_head, ws, off, s);
    if (e != hipSuccess) return hip_status(e);
  }
  return NABLA_OK;
}

}  // extern "C"
