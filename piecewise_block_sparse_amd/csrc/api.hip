// C ABI of libpisa: argument validation on the host, then kernel launches on
// the caller's stream.  Declared in include/pisa.h.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "launch.hpp"
#include "pisa.h"

namespace {

thread_local char g_err[256] = "";

pisa_status fail(pisa_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
pisa_status fail(pisa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

pisa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return PISA_OK;
  return fail(PISA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Shape rules shared by every call.  Returns PISA_OK and fills bh / nb.
pisa_status check_shape(const pisa_shape* s, int* bh, int* nb) {
  if (!s) return fail(PISA_ERR_NULL, "shape is NULL");
  if (s->dtype != PISA_DTYPE_BF16 && s->dtype != PISA_DTYPE_FP32)
    return fail(PISA_ERR_DTYPE, "unknown dtype %d", s->dtype);
  if (s->batch <= 0 || s->heads <= 0 || s->seq_len <= 0)
    return fail(PISA_ERR_SHAPE, "batch, heads and seq_len must be positive");
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(PISA_ERR_SHAPE, "head_dim %d not in {64, 128}", s->head_dim);
  if (s->block != 64 && s->block != 128)
    return fail(PISA_ERR_SHAPE, "block %d not in {64, 128}", s->block);
  if (s->seq_len % s->block != 0)
    return fail(PISA_ERR_SHAPE, "seq_len %d is not a multiple of block %d (pad per modality)",
                s->seq_len, s->block);
  const long long n = (long long)s->seq_len / s->block;
  if (n > pisa::kMaxBlocks)
    return fail(PISA_ERR_SHAPE, "seq_len / block = %lld exceeds %d blocks", n, pisa::kMaxBlocks);
  const long long b = (long long)s->batch * s->heads;
  if (b * n >= (1LL << 31))
    return fail(PISA_ERR_SHAPE, "batch * heads * blocks must stay below 2^31");
  // the Hbar reduction launches (d / 32)^2 <= 16 workgroups per head
  if (b >= (1LL << 27)) return fail(PISA_ERR_SHAPE, "batch * heads must stay below 2^27");
  *bh = (int)b;
  *nb = (int)n;
  return PISA_OK;
}

// Workspace of pisa_precompute_noalloc: a static device array, one copy per
// GPU, held until the process ends.  Host code never uses its name as an
// address: the device address of each GPU's copy comes from
// hipGetSymbolAddress, called once per device with that device current.
constexpr size_t kScratchBytes = PISA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];                 // device address of `scratch` per device

// The current device's copy of `scratch` (looked up on the first call there).
pisa_status scratch_for_current_device(void** ptr) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "pisa_precompute_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PISA_ERR_HIP, "pisa_precompute_noalloc: device %d above the %d the library tracks", dev,
                kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t g = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (g != hipSuccess) return hip_status(g, "pisa_precompute_noalloc: hipGetSymbolAddress");
    if (!p) return fail(PISA_ERR_HIP, "pisa_precompute_noalloc: no device address for the scratch array");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return PISA_OK;
}

}  // namespace

extern "C" {

int32_t pisa_version(void) { return PISA_VERSION; }

const char* pisa_status_string(int32_t status) {
  switch (status) {
    case PISA_OK: return "ok";
    case PISA_ERR_NULL: return "null pointer argument";
    case PISA_ERR_SHAPE: return "unsupported or inconsistent shape";
    case PISA_ERR_ARG: return "invalid argument";
    case PISA_ERR_DTYPE: return "unknown element type";
    case PISA_ERR_WORKSPACE: return "workspace too small";
    case PISA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* pisa_last_error(void) { return g_err; }

size_t pisa_workspace_size(const pisa_shape* shape) {
  int bh = 0, nb = 0;
  if (check_shape(shape, &bh, &nb) != PISA_OK) return 0;
  return shape->dtype == PISA_DTYPE_BF16 ? pisa::stats_workspace_bf16(bh, nb, shape->head_dim, shape->block)
                                         : pisa::stats_workspace_f32(bh, nb, shape->head_dim);
}

size_t pisa_packed_size(const pisa_shape* shape) {
  int bh = 0, nb = 0;
  if (check_shape(shape, &bh, &nb) != PISA_OK || shape->dtype != PISA_DTYPE_BF16) return 0;
  return pisa::stats_packed_bytes(bh, nb, shape->head_dim, shape->block);
}

pisa_status pisa_precompute(const pisa_shape* shape, const void* K, const void* V,
                            const pisa_stats* out, void* workspace, size_t workspace_bytes,
                            void* stream) {
  g_err[0] = 0;
  int bh = 0, nb = 0;
  pisa_status st = check_shape(shape, &bh, &nb);
  if (st != PISA_OK) return st;
  if (!K || !V || !out) return fail(PISA_ERR_NULL, "K, V and out are required");
  if (!out->centroid || !out->vsum || !out->Hbar || !out->M)
    return fail(PISA_ERR_NULL, "centroid, vsum, Hbar and M outputs are required");
  const bool bf = shape->dtype == PISA_DTYPE_BF16;
  if (!bf && out->Ht) return fail(PISA_ERR_ARG, "Ht (bf16 H_j^T) is for bf16 inputs only");
  if (out->m_norm != PISA_NORM_FROBENIUS && out->m_norm != PISA_NORM_SPECTRAL)
    return fail(PISA_ERR_ARG, "unknown m_norm %d", out->m_norm);
  const bool spectral = out->m_norm == PISA_NORM_SPECTRAL;
  if (spectral && bf && !out->H)
    return fail(PISA_ERR_NULL, "the spectral M_j with bf16 inputs needs the H output");
  const bool needs_ws = bf || out->H == nullptr;
  if (needs_ws) {
    const size_t need = pisa_workspace_size(shape);
    if (!workspace) return fail(PISA_ERR_NULL, "workspace of %zu bytes is required", need);
    if (workspace_bytes < need)
      return fail(PISA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  }
  pisa::StatsArgs a{K, V, out->centroid, out->vsum, out->H, out->Hbar, out->M,
                    bf ? out->packed : nullptr, bf ? out->Ht : nullptr, workspace,
                    spectral ? 1 : 0, bh, nb, shape->head_dim, shape->block, shape->seq_lens,
                    shape->heads, (hipStream_t)stream};
  return hip_status(bf ? pisa::launch_stats_bf16(a) : pisa::launch_stats_f32(a), "pisa_precompute");
}

pisa_status pisa_precompute_noalloc(const pisa_shape* shape, const void* K, const void* V,
                                    const pisa_stats* out, void* stream) {
  g_err[0] = 0;
  int bh = 0, nb = 0;
  pisa_status st = check_shape(shape, &bh, &nb);
  if (st != PISA_OK) return st;
  if (!K || !V || !out) return fail(PISA_ERR_NULL, "K, V and out are required");
  const size_t need = pisa_workspace_size(shape);
  if (need > kScratchBytes)
    return fail(PISA_ERR_WORKSPACE,
                "this shape needs %zu bytes of workspace, above the %zu bytes of "
                "pisa_precompute_noalloc's static scratch: use pisa_precompute with a workspace",
                need, kScratchBytes);
  void* ws = nullptr;
  st = scratch_for_current_device(&ws);
  if (st != PISA_OK) return st;
  return pisa_precompute(shape, K, V, out, ws, kScratchBytes, stream);
}

pisa_status pisa_route(const pisa_shape* shape, const void* Q, const float* centroid,
                       const float* M, int32_t k, double scale, double lambda, int32_t* idx,
                       void* stream) {
  g_err[0] = 0;
  int bh = 0, nb = 0;
  pisa_status st = check_shape(shape, &bh, &nb);
  if (st != PISA_OK) return st;
  if (!Q || !centroid || !M || !idx) return fail(PISA_ERR_NULL, "Q, centroid, M and idx are required");
  if (k < 1 || k > nb) return fail(PISA_ERR_ARG, "k=%d outside [1, %d]", k, nb);
  if (!std::isfinite(scale) || !std::isfinite(lambda))
    return fail(PISA_ERR_ARG, "scale and lambda must be finite");
  pisa::RouteArgs a{Q, centroid, M, k, scale, lambda, idx, bh, nb, shape->head_dim, shape->block,
                    shape->seq_lens, shape->heads, (hipStream_t)stream};
  const bool bf = shape->dtype == PISA_DTYPE_BF16;
  return hip_status(bf ? pisa::launch_route_bf16(a) : pisa::launch_route_f32(a), "pisa_route");
}

pisa_status pisa_attention(const pisa_shape* shape, const void* Q, const void* K,
                           const void* V, const int32_t* idx, int32_t kmax,
                           const pisa_stats* stats, int32_t mode, float scale, void* O,
                           void* stream) {
  g_err[0] = 0;
  int bh = 0, nb = 0;
  pisa_status st = check_shape(shape, &bh, &nb);
  if (st != PISA_OK) return st;
  if (!Q || !K || !V || !idx || !O) return fail(PISA_ERR_NULL, "Q, K, V, idx and O are required");
  if (mode != PISA_MODE_APPROX && mode != PISA_MODE_DROP && mode != PISA_MODE_ZEROTH &&
      mode != PISA_MODE_FIRST)
    return fail(PISA_ERR_ARG, "unknown mode %d", mode);
  if (kmax < 1 || kmax > nb) return fail(PISA_ERR_ARG, "kmax=%d outside [1, %d]", kmax, nb);
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(PISA_ERR_ARG, "scale must be finite and positive");
  const bool approx = mode != PISA_MODE_DROP;
  const bool bf = shape->dtype == PISA_DTYPE_BF16;
  const int order = mode == PISA_MODE_ZEROTH  ? pisa::kOrderZeroth
                    : mode == PISA_MODE_FIRST ? pisa::kOrderFirst
                                              : pisa::kOrderMixed;
  if (approx && (!stats || !stats->centroid || !stats->vsum))
    return fail(PISA_ERR_NULL, "modes other than DROP need stats centroid and vsum");
  if (mode == PISA_MODE_APPROX && !stats->Hbar)
    return fail(PISA_ERR_NULL, "APPROX mode needs stats Hbar");
  if (mode == PISA_MODE_FIRST && bf && (!stats->Ht || !stats->packed))
    return fail(PISA_ERR_NULL, "FIRST mode with bf16 inputs needs stats Ht and packed");
  if (mode == PISA_MODE_FIRST && !bf && !stats->H)
    return fail(PISA_ERR_NULL, "FIRST mode with fp32 inputs needs stats H");
  pisa::AttnArgs a{Q, K, V, idx, kmax,
                   approx ? stats->centroid : nullptr, approx ? stats->vsum : nullptr,
                   mode == PISA_MODE_APPROX ? stats->Hbar : nullptr,
                   (approx && bf) ? stats->packed : nullptr,
                   (mode == PISA_MODE_FIRST && bf) ? stats->Ht : nullptr,
                   (mode == PISA_MODE_FIRST && !bf) ? stats->H : nullptr,
                   approx ? 1 : 0, order, scale, O, bh, nb, shape->head_dim, shape->block,
                   shape->seq_lens, shape->heads, (hipStream_t)stream};
  return hip_status(bf ? pisa::launch_attn_bf16(a) : pisa::launch_attn_f32(a), "pisa_attention");
}

size_t pisa_attention_split_workspace_size(const pisa_shape* shape, int32_t kmax, int32_t max_blocks) {
  int bh = 0, nb = 0;
  if (check_shape(shape, &bh, &nb) != PISA_OK || shape->dtype != PISA_DTYPE_BF16) return 0;
  if (kmax < 1 || kmax > nb || max_blocks < 1) return 0;
  return pisa::attn_split_workspace(shape->head_dim, shape->block, bh, nb, kmax, max_blocks);
}

pisa_status pisa_attention_split(const pisa_shape* shape, const void* Q, const void* K,
                                 const void* V, const int32_t* idx, int32_t kmax,
                                 const pisa_stats* stats, int32_t mode, float scale,
                                 int32_t max_blocks, void* O, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  int bh = 0, nb = 0;
  pisa_status st = check_shape(shape, &bh, &nb);
  if (st != PISA_OK) return st;
  if (shape->dtype != PISA_DTYPE_BF16)
    return fail(PISA_ERR_DTYPE, "split work items are built for bf16 inputs");
  if (!Q || !K || !V || !idx || !O) return fail(PISA_ERR_NULL, "Q, K, V, idx and O are required");
  if (mode != PISA_MODE_APPROX && mode != PISA_MODE_DROP && mode != PISA_MODE_ZEROTH)
    return fail(PISA_ERR_ARG, "mode %d: split work items run APPROX, DROP or ZEROTH", mode);
  if (kmax < 1 || kmax > nb) return fail(PISA_ERR_ARG, "kmax=%d outside [1, %d]", kmax, nb);
  if (max_blocks < 1) return fail(PISA_ERR_ARG, "max_blocks=%d must be at least 1", max_blocks);
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(PISA_ERR_ARG, "scale must be finite and positive");
  const bool approx = mode != PISA_MODE_DROP;
  if (approx && (!stats || !stats->centroid || !stats->vsum))
    return fail(PISA_ERR_NULL, "modes other than DROP need stats centroid and vsum");
  if (mode == PISA_MODE_APPROX && !stats->Hbar)
    return fail(PISA_ERR_NULL, "APPROX mode needs stats Hbar");
  const size_t need = pisa_attention_split_workspace_size(shape, kmax, max_blocks);
  if (!workspace) return fail(PISA_ERR_NULL, "workspace of %zu bytes is required", need);
  {
    // the grid holds every part of every work item (a work item is a pair of
    // query blocks for 64-token blocks; items rounded up to a multiple of the
    // 8 XCDs)
    const long long qb = shape->block == 64 ? 2 : 1;
    const long long items = (long long)bh * ((nb + qb - 1) / qb);
    const long long most = std::min<long long>(nb, qb * kmax);
    const long long parts = std::min<long long>(32, std::max<long long>(1, (most + max_blocks - 1) / max_blocks));
    if ((items + 7) / 8 * 8 * parts >= (1LL << 31))
      return fail(PISA_ERR_SHAPE, "split attention: %lld work items x %lld parts exceed one grid", items, parts);
  }
  if (workspace_bytes < need)
    return fail(PISA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  const int order = mode == PISA_MODE_ZEROTH ? pisa::kOrderZeroth : pisa::kOrderMixed;
  pisa::AttnArgs a{Q, K, V, idx, kmax,
                   approx ? stats->centroid : nullptr, approx ? stats->vsum : nullptr,
                   mode == PISA_MODE_APPROX ? stats->Hbar : nullptr,
                   approx ? stats->packed : nullptr, nullptr, nullptr,
                   approx ? 1 : 0, order, scale, O, bh, nb, shape->head_dim, shape->block,
                   shape->seq_lens, shape->heads, (hipStream_t)stream,
                   nullptr, 0, 0.0, 0.0, nullptr, max_blocks, workspace};
  return hip_status(pisa::launch_attn_bf16(a), "pisa_attention_split");
}

pisa_status pisa_route_attention(const pisa_shape* shape, const void* Q, const void* K,
                                 const void* V, const pisa_stats* stats, int32_t k, double lambda,
                                 int32_t mode, double scale, int32_t* idx, void* O, int32_t form,
                                 void* stream) {
  g_err[0] = 0;
  int bh = 0, nb = 0;
  pisa_status st = check_shape(shape, &bh, &nb);
  if (st != PISA_OK) return st;
  if (!Q || !K || !V || !O || !stats || !stats->centroid || !stats->M)
    return fail(PISA_ERR_NULL, "Q, K, V, O and stats centroid and M are required");
  if (form != PISA_ROUTE_AUTO && form != PISA_ROUTE_IN_KERNEL && form != PISA_ROUTE_TWO_LAUNCH)
    return fail(PISA_ERR_ARG, "unknown form %d", form);
  if (form == PISA_ROUTE_TWO_LAUNCH && !idx)
    return fail(PISA_ERR_NULL, "the two-launch form needs idx for the selection");
  if (shape->dtype != PISA_DTYPE_BF16)
    return fail(PISA_ERR_DTYPE, "in-kernel routing is built for bf16 inputs");
  if (mode == PISA_MODE_FIRST)
    return fail(PISA_ERR_ARG, "FIRST mode: use pisa_route, then pisa_attention");
  if (mode != PISA_MODE_APPROX && mode != PISA_MODE_DROP && mode != PISA_MODE_ZEROTH)
    return fail(PISA_ERR_ARG, "unknown mode %d", mode);
  if (k < 1 || k > nb) return fail(PISA_ERR_ARG, "k=%d outside [1, %d]", k, nb);
  if (!std::isfinite(scale) || !(scale > 0.0) || !((float)scale > 0.f) || !std::isfinite((float)scale))
    return fail(PISA_ERR_ARG, "scale must be finite and positive");
  if (!std::isfinite(lambda)) return fail(PISA_ERR_ARG, "lambda must be finite");
  const bool approx = mode != PISA_MODE_DROP;
  if (approx && !stats->vsum) return fail(PISA_ERR_NULL, "modes other than DROP need stats vsum");
  if (mode == PISA_MODE_APPROX && !stats->Hbar)
    return fail(PISA_ERR_NULL, "APPROX mode needs stats Hbar");
  const int maxnb = pisa::fused_route_max_blocks(shape->head_dim, shape->block);
  bool two = form == PISA_ROUTE_TWO_LAUNCH;
  if (form == PISA_ROUTE_AUTO && idx) {
    // in-kernel routing only while the work items fit one round of workgroups
    const int resident = pisa::fused_route_resident(shape->head_dim, shape->block);
    two = nb > maxnb ||
          (resident > 0 && pisa::fused_route_items(shape->head_dim, shape->block, bh, nb) > resident);
  }
  if (!two && nb > maxnb)
    return fail(PISA_ERR_SHAPE, "nb=%d above %d for in-kernel routing at d=%d, block=%d: "
                "use pisa_route, then pisa_attention", nb, maxnb, shape->head_dim, shape->block);
  const int order = mode == PISA_MODE_ZEROTH ? pisa::kOrderZeroth : pisa::kOrderMixed;
  if (two) {
    // pisa_route into idx, then pisa_attention on it (scale as the in-kernel form uses it)
    pisa::RouteArgs r{Q, stats->centroid, stats->M, k, scale, lambda, idx, bh, nb, shape->head_dim,
                      shape->block, shape->seq_lens, shape->heads, (hipStream_t)stream};
    const pisa_status rs = hip_status(pisa::launch_route_bf16(r), "pisa_route_attention (routing)");
    if (rs != PISA_OK) return rs;
    pisa::AttnArgs a{Q, K, V, idx, k,
                     approx ? stats->centroid : nullptr, approx ? stats->vsum : nullptr,
                     mode == PISA_MODE_APPROX ? stats->Hbar : nullptr,
                     approx ? stats->packed : nullptr, nullptr, nullptr,
                     approx ? 1 : 0, order, (float)scale, O, bh, nb, shape->head_dim, shape->block,
                     shape->seq_lens, shape->heads, (hipStream_t)stream};
    return hip_status(pisa::launch_attn_bf16(a), "pisa_route_attention (attention)");
  }
  pisa::AttnArgs a{Q, K, V, nullptr, k,
                   stats->centroid, approx ? stats->vsum : nullptr,
                   mode == PISA_MODE_APPROX ? stats->Hbar : nullptr,
                   approx ? stats->packed : nullptr, nullptr, nullptr,
                   approx ? 1 : 0, order, (float)scale, O, bh, nb, shape->head_dim, shape->block,
                   shape->seq_lens, shape->heads, (hipStream_t)stream,
                   stats->M, k, scale, lambda, idx};
  return hip_status(pisa::launch_attn_bf16(a), "pisa_route_attention");
}

}  // extern "C"
