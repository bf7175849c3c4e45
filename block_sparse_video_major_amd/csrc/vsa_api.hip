// Host entry points of libvsa.so (the C ABI declared in include/vsa.h).
//
// Every entry point validates its arguments on the host and returns before
// anything is queued if they are invalid; otherwise it launches its kernels on
// the caller's stream and returns without synchronising.  No entry point
// allocates or frees memory.
#include <limits.h>
#include <math.h>

#include <algorithm>
#include <mutex>

#include "vsa_internal.h"

namespace {

using vsa::Geom;

int check_problem(const vsa_problem* p, bool need_table = true) {
  if (p == nullptr) return VSA_ERR_NULL;
  if (p->batch <= 0 || p->heads <= 0 || p->T <= 0 || p->H <= 0 || p->W <= 0 || p->ct <= 0 ||
      p->ch <= 0 || p->cw <= 0 || p->head_dim <= 0)
    return VSA_ERR_SHAPE;
  if (p->heads_kv < 0 || (p->heads_kv > 0 && p->heads % p->heads_kv)) return VSA_ERR_SHAPE;
  // a grid that does not divide into cubes is padded up to whole cubes
  const auto up = [](int64_t x, int64_t c) { return (x + c - 1) / c * c; };
  const int64_t n = up(p->T, p->ct) * up(p->H, p->ch) * up(p->W, p->cw);
  const int64_t vol = (int64_t)p->ct * p->ch * p->cw;
  const int64_t bh = (int64_t)p->batch * p->heads;
  if (n > INT32_MAX || vol > INT32_MAX || bh > INT32_MAX) return VSA_ERR_SHAPE;
  // every element index must fit comfortably in int64 and every launch grid in 2^31 blocks
  if (bh * n > ((int64_t)1 << 40)) return VSA_ERR_SHAPE;
  if (p->head_dim != 64 && p->head_dim != 128) return VSA_ERR_UNSUPPORTED;
  if (p->head_dim_v != 0 && p->head_dim_v != 64 && p->head_dim_v != 128) return VSA_ERR_UNSUPPORTED;
  if (p->cube_order != VSA_CUBES_RASTER && p->cube_order != VSA_CUBES_HILBERT) return VSA_ERR_UNSUPPORTED;
  if (p->cube_order == VSA_CUBES_HILBERT) {
    const int64_t sides[3] = {(p->T + (int64_t)p->ct - 1) / p->ct, (p->H + (int64_t)p->ch - 1) / p->ch,
                              (p->W + (int64_t)p->cw - 1) / p->cw};
    for (int64_t s : sides)
      if (s > 1024) return VSA_ERR_UNSUPPORTED;   // 10 bits per packed coordinate
    if (need_table && p->cube_coords == nullptr) return VSA_ERR_NULL;
  }
  return VSA_OK;
}

// Distance of cell (t, h, w) along the 3D Hilbert curve that fills the cube
// of side 2^bits (Skilling, "Programming the Hilbert curve", 2004).  From
// the coarsest level down, a coordinate whose bit is set at that level
// reflects the lower bits of t, otherwise t and that coordinate exchange
// their lower bits (undoing the sub-cubes' rotations and reflections); the
// three are then Gray-encoded together, and the distance takes their bits
// level by level from the top, t before h before w.
uint32_t hilbert_distance(uint32_t t, uint32_t h, uint32_t w, int bits) {
  uint32_t x[3] = {t, h, w};
  for (uint32_t level = 1u << (bits - 1); level > 1; level >>= 1) {
    const uint32_t low = level - 1;
    for (int i = 0; i < 3; ++i) {
      if (x[i] & level) {
        x[0] ^= low;
      } else {
        const uint32_t swap = (x[0] ^ x[i]) & low;
        x[0] ^= swap;
        x[i] ^= swap;
      }
    }
  }
  x[1] ^= x[0];
  x[2] ^= x[1];
  uint32_t flip = 0;
  for (uint32_t level = 1u << (bits - 1); level > 1; level >>= 1)
    if (x[2] & level) flip ^= level - 1;
  for (uint32_t& c : x) c ^= flip;
  uint32_t dist = 0;
  for (int b = bits - 1; b >= 0; --b)
    for (int i = 0; i < 3; ++i) dist = (dist << 1) | ((x[i] >> b) & 1u);
  return dist;
}

// out[c] = packed grid coordinates (t << 20 | h << 10 | w) of the c-th cube
// in the problem's cube order; every side at most 1024 (checked by the
// caller).  Sorted in place by curve distance: no allocation.
void fill_cube_table(const Geom& g, int order, int32_t* out) {
  int32_t c = 0;
  for (int32_t t = 0; t < g.gT; ++t)
    for (int32_t h = 0; h < g.gH; ++h)
      for (int32_t w = 0; w < g.gW; ++w) out[c++] = (t << 20) | (h << 10) | w;
  if (order == VSA_CUBES_RASTER) return;
  int bits = 1;
  while ((1 << bits) < std::max(g.gT, std::max(g.gH, g.gW))) ++bits;
  const auto dist = [bits](int32_t e) {
    return hilbert_distance((uint32_t)(e >> 20) & 1023u, (uint32_t)(e >> 10) & 1023u, (uint32_t)e & 1023u, bits);
  };
  std::sort(out, out + c, [&](int32_t a, int32_t b) { return dist(a) < dist(b); });
}

int check_dtype(int32_t dtype) {
  return (dtype == VSA_BF16 || dtype == VSA_F32) ? VSA_OK : VSA_ERR_UNSUPPORTED;
}

int hip_status(hipError_t e) { return e == hipSuccess ? VSA_OK : VSA_ERR_HIP; }

}  // namespace

extern "C" {

int vsa_abi_version(void) { return (3 << 16) | 3; }

int vsa_device_peak(int32_t device, int32_t* cu_count, int32_t* clock_khz, double* bf16_tflops) {
  int cus = 0, khz = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
      hipDeviceGetAttribute(&khz, hipDeviceAttributeClockRate, device) != hipSuccess)
    return VSA_ERR_HIP;
  if (cu_count) *cu_count = cus;
  if (clock_khz) *clock_khz = khz;
  if (bf16_tflops) *bf16_tflops = (double)cus * (double)khz * 1e3 * 4096.0 / 1e12;
  return VSA_OK;
}

const char* vsa_status_str(int status) {
  switch (status) {
    case VSA_OK: return "ok";
    case VSA_ERR_NULL: return "required pointer is NULL";
    case VSA_ERR_SHAPE: return "invalid shape (non-positive size, heads_kv not dividing heads, or too large)";
    case VSA_ERR_TOPK: return "top_k / max_kv_blocks outside [1, Nc]";
    case VSA_ERR_UNSUPPORTED: return "unsupported head_dim, dtype, cube volume, cube count or cube order";
    case VSA_ERR_HIP: return "HIP runtime error at launch";
    case VSA_ERR_LUT: return "invalid LUT";
    case VSA_ERR_WORKSPACE:
      return "workspace smaller than the workspace query reports (or, for the _noalloc entry point, needing more "
             "than VSA_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int vsa_perm_index(const vsa_problem* p, int32_t* perm_host) {
  int st = check_problem(p, false);
  if (st != VSA_OK) return st;
  if (perm_host == nullptr) return VSA_ERR_NULL;
  const Geom g = vsa::make_geom(*p);
  if (p->cube_order == VSA_CUBES_RASTER) {
    int64_t pos = 0;
    for (int ct_i = 0; ct_i < g.gT; ++ct_i)
      for (int ch_i = 0; ch_i < g.gH; ++ch_i)
        for (int cw_i = 0; cw_i < g.gW; ++cw_i)
          for (int lt = 0; lt < g.ct; ++lt)
            for (int lh = 0; lh < g.ch; ++lh)
              for (int lw = 0; lw < g.cw; ++lw) {
                const int64_t t = (int64_t)ct_i * g.ct + lt, h = (int64_t)ch_i * g.ch + lh,
                              w = (int64_t)cw_i * g.cw + lw;
                const bool real = t < g.T && h < g.H && w < g.W;
                perm_host[pos++] = real ? (int32_t)((t * g.H + h) * g.W + w) : -1;
              }
    return VSA_OK;
  }
  // The cube table goes into the first Nc entries; cubes are then expanded
  // from the last one down.  Cube c's vol positions start at c*vol >= c, so
  // entries of cubes not yet expanded are never overwritten first.
  fill_cube_table(g, p->cube_order, perm_host);
  for (int64_t c = g.Nc - 1; c >= 0; --c) {
    const int32_t e = perm_host[c];
    const int64_t ct_i = (e >> 20) & 1023, ch_i = (e >> 10) & 1023, cw_i = e & 1023;
    int64_t pos = c * g.vol;
    for (int lt = 0; lt < g.ct; ++lt)
      for (int lh = 0; lh < g.ch; ++lh)
        for (int lw = 0; lw < g.cw; ++lw) {
          const int64_t t = ct_i * g.ct + lt, h = ch_i * g.ch + lh, w = cw_i * g.cw + lw;
          const bool real = t < g.T && h < g.H && w < g.W;
          perm_host[pos++] = real ? (int32_t)((t * g.H + h) * g.W + w) : -1;
        }
  }
  return VSA_OK;
}

int vsa_cube_table(const vsa_problem* p, int32_t* coords_host) {
  int st = check_problem(p, false);
  if (st != VSA_OK) return st;
  if (coords_host == nullptr) return VSA_ERR_NULL;
  const Geom g = vsa::make_geom(*p);
  if (g.gT > 1024 || g.gH > 1024 || g.gW > 1024) return VSA_ERR_UNSUPPORTED;
  fill_cube_table(g, p->cube_order, coords_host);
  return VSA_OK;
}

int vsa_permute(const vsa_problem* p, int32_t dtype, const void* x_raster, void* x_cube, void* stream) {
  int st = check_problem(p);
  if (st == VSA_OK) st = check_dtype(dtype);
  if (st != VSA_OK) return st;
  if (x_raster == nullptr || x_cube == nullptr) return VSA_ERR_NULL;
  const Geom g = vsa::make_geom(*p);
  return hip_status(vsa::launch_reorder(g, dtype, x_raster, x_cube, true, (hipStream_t)stream));
}

int vsa_unpermute(const vsa_problem* p, int32_t dtype, const void* x_cube, void* x_raster, void* stream) {
  int st = check_problem(p);
  if (st == VSA_OK) st = check_dtype(dtype);
  if (st != VSA_OK) return st;
  if (x_raster == nullptr || x_cube == nullptr) return VSA_ERR_NULL;
  const Geom g = vsa::make_geom(*p);
  return hip_status(vsa::launch_reorder(g, dtype, x_cube, x_raster, false, (hipStream_t)stream));
}

int vsa_pool(const vsa_problem* p, int32_t dtype, const void* x_cube, float* xc, void* stream) {
  int st = check_problem(p);
  if (st == VSA_OK) st = check_dtype(dtype);
  if (st != VSA_OK) return st;
  if (x_cube == nullptr || xc == nullptr) return VSA_ERR_NULL;
  const Geom g = vsa::make_geom(*p);
  return hip_status(vsa::launch_pool(g, dtype, x_cube, xc, (hipStream_t)stream));
}

int vsa_permute_pool(const vsa_problem* p, int32_t dtype, const void* x_raster, void* x_cube, float* xc,
                     void* stream) {
  int st = check_problem(p);
  if (st == VSA_OK) st = check_dtype(dtype);
  if (st != VSA_OK) return st;
  if (x_raster == nullptr || xc == nullptr) return VSA_ERR_NULL;   // x_cube == NULL: pool only
  const Geom g = vsa::make_geom(*p);
  return hip_status(vsa::launch_permute_pool(g, dtype, x_raster, x_cube, xc, (hipStream_t)stream));
}

int vsa_coarse_topk(const vsa_problem* p, int32_t top_k, const float* qc, const float* kc, const float* vc,
                    int32_t* kv_block_idx, int32_t* valid_block_num, float* oc, void* stream) {
  int st = check_problem(p);
  if (st != VSA_OK) return st;
  if (qc == nullptr || kc == nullptr || kv_block_idx == nullptr || valid_block_num == nullptr)
    return VSA_ERR_NULL;
  if (oc != nullptr && vc == nullptr) return VSA_ERR_NULL;
  const Geom g = vsa::make_geom(*p);
  if (g.Nc > vsa::kMaxCoarseCubes) return VSA_ERR_UNSUPPORTED;
  if (top_k < 1 || top_k > g.Nc) return VSA_ERR_TOPK;
  return hip_status(vsa::launch_coarse_topk(g, top_k, qc, kc, vc, kv_block_idx, valid_block_num, oc,
                                            (hipStream_t)stream));
}

namespace {
int sparse_attn_fwd_common(const vsa_problem* p, const void* q, const void* k, const void* v,
                           const int32_t* kv_block_idx, const int32_t* valid_block_num, int32_t max_kv_blocks,
                           const float* oc, const void* gate_c, const void* gate_f, void* out, float* lse,
                           int out_order, void* stream) {
  int st = check_problem(p);
  if (st != VSA_OK) return st;
  if (q == nullptr || k == nullptr || v == nullptr || kv_block_idx == nullptr || valid_block_num == nullptr ||
      out == nullptr)
    return VSA_ERR_NULL;
  if (gate_c != nullptr && oc == nullptr) return VSA_ERR_NULL;
  const Geom g = vsa::make_geom(*p);
  if (g.vol != 64) return VSA_ERR_UNSUPPORTED;
  if (max_kv_blocks < 1 || max_kv_blocks > g.Nc) return VSA_ERR_TOPK;
  if (g.Dv != g.D) {   // value head size of its own: the four-wavefront kernel
    if (!vsa::sparse_attn_fwd_dv_fits(g, max_kv_blocks)) return VSA_ERR_UNSUPPORTED;
    return hip_status(vsa::launch_sparse_attn_fwd_dv(g, q, k, v, kv_block_idx, valid_block_num, max_kv_blocks, oc,
                                                     gate_c, gate_f, out, lse, out_order, (hipStream_t)stream));
  }
  if (!vsa::sparse_attn_fwd_fits(g, max_kv_blocks)) return VSA_ERR_UNSUPPORTED;
  return hip_status(vsa::launch_sparse_attn_fwd(g, q, k, v, kv_block_idx, valid_block_num, max_kv_blocks, oc,
                                                gate_c, gate_f, out, lse, out_order, (hipStream_t)stream));
}
}  // namespace

int vsa_sparse_attn_fwd(const vsa_problem* p, const void* q, const void* k, const void* v,
                        const int32_t* kv_block_idx, const int32_t* valid_block_num, int32_t max_kv_blocks,
                        const float* oc, const void* gate_c, const void* gate_f, void* out, float* lse,
                        void* stream) {
  return sparse_attn_fwd_common(p, q, k, v, kv_block_idx, valid_block_num, max_kv_blocks, oc, gate_c, gate_f,
                                out, lse, 0, stream);
}

int vsa_sparse_attn_fwd_raster(const vsa_problem* p, const void* q, const void* k, const void* v,
                               const int32_t* kv_block_idx, const int32_t* valid_block_num,
                               int32_t max_kv_blocks, const float* oc, const void* gate_c, const void* gate_f,
                               void* out, float* lse, void* stream) {
  return sparse_attn_fwd_common(p, q, k, v, kv_block_idx, valid_block_num, max_kv_blocks, oc, gate_c, gate_f,
                                out, lse, 1, stream);
}

int vsa_sparse_attn_fwd_gather(const vsa_problem* p, const void* q, const void* k, const void* v,
                               const int32_t* kv_block_idx, const int32_t* valid_block_num,
                               int32_t max_kv_blocks, const float* oc, const void* gate_c, const void* gate_f,
                               void* out, float* lse, void* stream) {
  int st = check_problem(p);
  if (st != VSA_OK) return st;
  if (q == nullptr || k == nullptr || v == nullptr || kv_block_idx == nullptr || valid_block_num == nullptr ||
      out == nullptr)
    return VSA_ERR_NULL;
  if (gate_c != nullptr && oc == nullptr) return VSA_ERR_NULL;
  const Geom g = vsa::make_geom(*p);
  if (max_kv_blocks < 1 || max_kv_blocks > g.Nc) return VSA_ERR_TOPK;
  if (!vsa::sparse_attn_fwd_gather_fits(g, max_kv_blocks)) return VSA_ERR_UNSUPPORTED;
  return hip_status(vsa::launch_sparse_attn_fwd(g, q, k, v, kv_block_idx, valid_block_num, max_kv_blocks, oc,
                                                gate_c, gate_f, out, lse, 1, (hipStream_t)stream, true));
}

int vsa_sparse_attn_fwd_bnhd(const vsa_problem* p, const void* q, const void* k, const void* v,
                             const int32_t* kv_block_idx, const int32_t* valid_block_num, int32_t max_kv_blocks,
                             const float* oc, const void* gate_c, const void* gate_f, void* out, float* lse,
                             void* stream) {
  return sparse_attn_fwd_common(p, q, k, v, kv_block_idx, valid_block_num, max_kv_blocks, oc, gate_c, gate_f,
                                out, lse, 2, stream);
}

int vsa_permute_bnhd(const vsa_problem* p, int32_t dtype, const void* x_bnhd, void* x_cube, void* stream) {
  int st = check_problem(p);
  if (st == VSA_OK) st = check_dtype(dtype);
  if (st != VSA_OK) return st;
  if (x_bnhd == nullptr || x_cube == nullptr) return VSA_ERR_NULL;
  const Geom g = vsa::make_geom(*p);
  return hip_status(vsa::launch_reorder(g, dtype, x_bnhd, x_cube, true, (hipStream_t)stream, vsa::kBNHD));
}

int vsa_permute_pool_bnhd(const vsa_problem* p, int32_t dtype, const void* x_bnhd, void* x_cube, float* xc,
                          void* stream) {
  int st = check_problem(p);
  if (st == VSA_OK) st = check_dtype(dtype);
  if (st != VSA_OK) return st;
  if (x_bnhd == nullptr || xc == nullptr) return VSA_ERR_NULL;   // x_cube == NULL: pool only
  const Geom g = vsa::make_geom(*p);
  return hip_status(vsa::launch_permute_pool(g, dtype, x_bnhd, x_cube, xc, (hipStream_t)stream, vsa::kBNHD));
}

namespace {
int sparse_attn_bwd_check(const vsa_problem* p, int32_t max_kv_blocks, bool need_table = true) {
  int st = check_problem(p, need_table);
  if (st != VSA_OK) return st;
  const Geom g = vsa::make_geom(*p);
  if (g.vol != 64) return VSA_ERR_UNSUPPORTED;
  if (max_kv_blocks < 1 || max_kv_blocks > g.Nc) return VSA_ERR_TOPK;
  if (!vsa::sparse_attn_bwd_fits(g, max_kv_blocks)) return VSA_ERR_UNSUPPORTED;
  return VSA_OK;
}
}  // namespace

int vsa_sparse_attn_bwd_workspace_size(const vsa_problem* p, int32_t max_kv_blocks, size_t* bytes) {
  if (bytes == nullptr) return VSA_ERR_NULL;
  const int st = sparse_attn_bwd_check(p, max_kv_blocks, false);
  if (st != VSA_OK) return st;
  *bytes = vsa::sparse_attn_bwd_workspace(vsa::make_geom(*p), max_kv_blocks);
  return VSA_OK;
}

int vsa_sparse_attn_bwd(const vsa_problem* p, const void* q, const void* k, const void* v,
                        const int32_t* kv_block_idx, const int32_t* valid_block_num, int32_t max_kv_blocks,
                        const void* o, const float* lse, const void* d_o, float* dq, float* dk, float* dv,
                        void* workspace, size_t workspace_bytes, void* stream) {
  const int st = sparse_attn_bwd_check(p, max_kv_blocks);
  if (st != VSA_OK) return st;
  if (q == nullptr || k == nullptr || v == nullptr || kv_block_idx == nullptr || valid_block_num == nullptr ||
      o == nullptr || lse == nullptr || d_o == nullptr || dq == nullptr || dk == nullptr || dv == nullptr ||
      workspace == nullptr)
    return VSA_ERR_NULL;
  const Geom g = vsa::make_geom(*p);
  if (workspace_bytes < vsa::sparse_attn_bwd_workspace(g, max_kv_blocks)) return VSA_ERR_WORKSPACE;
  return hip_status(vsa::launch_sparse_attn_bwd(g, q, k, v, kv_block_idx, valid_block_num, max_kv_blocks, o, lse,
                                                d_o, dq, dk, dv, workspace, (hipStream_t)stream));
}

namespace {
// Workspace of vsa_sparse_attn_bwd_noalloc: one fixed array per GPU, held
// until the process ends.  Host code only ever uses the device address that
// hipGetSymbolAddress reports for the current device (the array's name in
// host code is a host-side stand-in, not a device address).
static __device__ __align__(256) unsigned char scratch[VSA_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up on its first use on
// that device (with that device current) and kept.
hipError_t scratch_on_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    scratch_ptr[dev] = ptr;
  }
  *out = scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

int vsa_sparse_attn_bwd_noalloc(const vsa_problem* p, const void* q, const void* k, const void* v,
                                const int32_t* kv_block_idx, const int32_t* valid_block_num,
                                int32_t max_kv_blocks, const void* o, const float* lse, const void* d_o, float* dq,
                                float* dk, float* dv, void* stream) {
  const int st = sparse_attn_bwd_check(p, max_kv_blocks);
  if (st != VSA_OK) return st;
  if (q == nullptr || k == nullptr || v == nullptr || kv_block_idx == nullptr || valid_block_num == nullptr ||
      o == nullptr || lse == nullptr || d_o == nullptr || dq == nullptr || dk == nullptr || dv == nullptr)
    return VSA_ERR_NULL;
  const Geom g = vsa::make_geom(*p);
  if (vsa::sparse_attn_bwd_workspace(g, max_kv_blocks) > (size_t)VSA_NOALLOC_SCRATCH_BYTES)
    return VSA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (scratch_on_current_device(&ws) != hipSuccess) return VSA_ERR_HIP;
  // every byte of the workspace the kernels read is written by them first
  // (per-token records, list counts, offsets and the list itself), so the
  // previous call's contents need no clearing
  return hip_status(vsa::launch_sparse_attn_bwd(g, q, k, v, kv_block_idx, valid_block_num, max_kv_blocks, o, lse,
                                                d_o, dq, dk, dv, ws, (hipStream_t)stream));
}

int vsa_combine(const vsa_problem* p, const void* o_f, const float* oc, const void* gate_c, const void* gate_f,
                void* out, void* stream) {
  int st = check_problem(p);
  if (st != VSA_OK) return st;
  if (o_f == nullptr || out == nullptr) return VSA_ERR_NULL;
  if (gate_c != nullptr && oc == nullptr) return VSA_ERR_NULL;
  const Geom g = vsa::make_geom(*p);
  return hip_status(vsa::launch_combine(g, o_f, oc, gate_c, gate_f, out, (hipStream_t)stream));
}

int vsa_combine_bwd(const vsa_problem* p, const void* dout, const void* o_f, const float* oc, const void* gate_c,
                    const void* gate_f, void* d_of, float* d_oc, float* d_gate_c, float* d_gate_f, void* stream) {
  int st = check_problem(p);
  if (st != VSA_OK) return st;
  if (dout == nullptr || d_of == nullptr || d_oc == nullptr) return VSA_ERR_NULL;
  if (gate_f != nullptr && (o_f == nullptr || d_gate_f == nullptr)) return VSA_ERR_NULL;
  if (gate_c != nullptr && (oc == nullptr || d_gate_c == nullptr)) return VSA_ERR_NULL;
  const Geom g = vsa::make_geom(*p);
  return hip_status(vsa::launch_combine_bwd(g, dout, o_f, oc, gate_c, gate_f, d_of, d_oc, d_gate_c, d_gate_f,
                                            (hipStream_t)stream));
}

int vsa_coarse_bwd_workspace_size(const vsa_problem* p, size_t* bytes) {
  int st = check_problem(p, false);
  if (st != VSA_OK) return st;
  if (bytes == nullptr) return VSA_ERR_NULL;
  const Geom g = vsa::make_geom(*p);
  if (g.Nc > vsa::kMaxCoarseCubes) return VSA_ERR_UNSUPPORTED;
  *bytes = vsa::coarse_bwd_workspace(g);
  return VSA_OK;
}

int vsa_coarse_bwd(const vsa_problem* p, const float* qc, const float* kc, const float* vc, const float* oc,
                   const float* d_oc, float* dqc, float* dkc, float* dvc, void* workspace, size_t workspace_bytes,
                   void* stream) {
  int st = check_problem(p);
  if (st != VSA_OK) return st;
  if (qc == nullptr || kc == nullptr || vc == nullptr || oc == nullptr || d_oc == nullptr || dqc == nullptr ||
      dkc == nullptr || dvc == nullptr || workspace == nullptr)
    return VSA_ERR_NULL;
  const Geom g = vsa::make_geom(*p);
  if (g.Nc > vsa::kMaxCoarseCubes) return VSA_ERR_UNSUPPORTED;
  if (workspace_bytes < vsa::coarse_bwd_workspace(g)) return VSA_ERR_WORKSPACE;
  return hip_status(vsa::launch_coarse_bwd(g, qc, kc, vc, oc, d_oc, dqc, dkc, dvc, workspace, (hipStream_t)stream));
}

int vsa_pool_unpermute_bwd(const vsa_problem* p, const float* dx_cube, const float* dxc, float* dx_raster,
                           void* stream) {
  int st = check_problem(p);
  if (st != VSA_OK) return st;
  if (dx_cube == nullptr || dx_raster == nullptr) return VSA_ERR_NULL;
  const Geom g = vsa::make_geom(*p);
  return hip_status(vsa::launch_pool_unpermute_bwd(g, dx_cube, dxc, dx_raster, (hipStream_t)stream));
}

int vsa_pool_unpermute_bwd_bnhd(const vsa_problem* p, const float* dx_cube, const float* dxc, float* dx_bnhd,
                                void* stream) {
  int st = check_problem(p);
  if (st != VSA_OK) return st;
  if (dx_cube == nullptr || dx_bnhd == nullptr) return VSA_ERR_NULL;
  const Geom g = vsa::make_geom(*p);
  return hip_status(vsa::launch_pool_unpermute_bwd(g, dx_cube, dxc, dx_bnhd, (hipStream_t)stream, vsa::kBNHD));
}

int vsa_check_lut(const vsa_problem* p, const int32_t* kv_block_idx, const int32_t* valid_block_num,
                  int32_t max_kv_blocks, int32_t* bad_rows, void* stream) {
  int st = check_problem(p);
  if (st != VSA_OK) return st;
  if (kv_block_idx == nullptr || valid_block_num == nullptr || bad_rows == nullptr) return VSA_ERR_NULL;
  const Geom g = vsa::make_geom(*p);
  if (max_kv_blocks < 1 || max_kv_blocks > g.Nc) return VSA_ERR_TOPK;
  return hip_status(vsa::launch_check_lut(g, kv_block_idx, valid_block_num, max_kv_blocks, bad_rows,
                                          (hipStream_t)stream));
}

int vsa_mask_to_lut(const vsa_problem* p, const uint8_t* mask, int32_t max_kv_blocks, int32_t* kv_block_idx,
                    int32_t* valid_block_num, int32_t* overflow_rows, void* stream) {
  int st = check_problem(p);
  if (st != VSA_OK) return st;
  if (mask == nullptr || kv_block_idx == nullptr || valid_block_num == nullptr || overflow_rows == nullptr)
    return VSA_ERR_NULL;
  const Geom g = vsa::make_geom(*p);
  if (max_kv_blocks < 1 || max_kv_blocks > g.Nc) return VSA_ERR_TOPK;
  return hip_status(vsa::launch_mask_to_lut(g, mask, max_kv_blocks, kv_block_idx, valid_block_num, overflow_rows,
                                            (hipStream_t)stream));
}

}  // extern "C"
