// Host entry points of the decode-attention C ABI (see include/kvq.h):
// argument validation, the split plan, workspace layout, the cooperative
// launch and the statistics readback. The kernels live in kvq_gqa.hip.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "kvq.h"
#include "kvq_internal.h"

namespace kvq {
size_t gqa_lds_bytes(int G, int P);
const void* gqa_kernel(int fmt, int G);
}  // namespace kvq

namespace {

using kvq::WsHeader;
using kvq::WsLayout;

struct DeviceInfo {
  int cus = 0;
  int max_lds = 0;
};

// Per-device cache of the compute-unit count and the LDS limit.
DeviceInfo device_info(int dev) {
  static std::mutex mu;
  static DeviceInfo cache[64];
  std::lock_guard<std::mutex> lock(mu);
  if (dev < 0 || dev >= 64) return DeviceInfo{};
  if (cache[dev].cus == 0) {
    int cus = 0, lds = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return DeviceInfo{};
    if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) return DeviceInfo{};
    cache[dev].cus = cus;
    cache[dev].max_lds = lds;
  }
  return cache[dev];
}

struct Plan {
  int S = 0, P = 0, G = 0, Dv = 0;
  size_t lds = 0;
  int nwg = 0;
  WsLayout ws{};
};

bool is_gqa_fmt(int fmt) { return fmt == KVQ_Q8_0 || fmt == KVQ_Q4_0 || fmt == KVQ_LUT3; }

// Validate shapes shared by every entry point and pick splits.
int32_t make_plan(int32_t fmt, const kvq_cache* k, const kvq_launch* l, int32_t ctx_len, Plan* plan) {
  if (!k || !l || !plan) return KVQ_ERR_ARG;
  if (fmt < KVQ_Q8_0 || fmt > KVQ_FP8_B128) return KVQ_ERR_ARG;
  if (k->batch <= 0 || k->heads <= 0 || k->dim <= 0 || k->capacity <= 0) return KVQ_ERR_ARG;
  if (l->q_heads <= 0 || l->q_heads % k->heads) return KVQ_ERR_ARG;
  if (l->q_dtype != KVQ_Q_F32 && l->q_dtype != KVQ_Q_BF16) return KVQ_ERR_ARG;
  if (ctx_len < 1 || ctx_len > k->capacity) return KVQ_ERR_RANGE;
  if (!is_gqa_fmt(fmt)) return KVQ_ERR_UNSUPPORTED;
  if (k->dim != 128) return KVQ_ERR_UNSUPPORTED;
  const int G = l->q_heads / k->heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return KVQ_ERR_UNSUPPORTED;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return KVQ_ERR_LAUNCH;
  const DeviceInfo di = device_info(dev);
  if (di.cus <= 0) return KVQ_ERR_LAUNCH;

  const int64_t BG = int64_t(k->batch) * k->heads;
  int S;
  if (l->splits > 0) {
    S = l->splits;
  } else {
    const int64_t target = di.cus;                        // one 16-wave workgroup per CU
    int64_t s = target / BG;
    if (s < 1) s = 1;
    const int64_t most = (ctx_len + kvq::kChunk - 1) / kvq::kChunk;
    if (s > most) s = most;
    S = int(s);
  }
  int P = (ctx_len + S - 1) / S;
  P = (P + kvq::kChunk - 1) / kvq::kChunk * kvq::kChunk;
  S = (ctx_len + P - 1) / P;                             // drop splits that would be empty
  if (P > 8192) return KVQ_ERR_UNSUPPORTED;              // per-split counts are packed in 14/18 bits
  const size_t lds = kvq::gqa_lds_bytes(G, P);
  if (lds > size_t(di.max_lds)) return KVQ_ERR_UNSUPPORTED;
  if (S > 2048 || BG * S > (int64_t(1) << 30)) return KVQ_ERR_UNSUPPORTED;

  plan->S = S;
  plan->P = P;
  plan->G = G;
  plan->Dv = 128;
  plan->lds = lds;
  plan->nwg = int(BG * S);
  plan->ws = kvq::ws_layout(k->batch, k->heads, l->q_heads, S, plan->Dv);
  return KVQ_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" const char* kvq_strerror(int32_t code) {
  switch (code) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_ARG: return "invalid argument";
    case KVQ_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case KVQ_ERR_RANGE: return "value out of range";
    case KVQ_ERR_NONFINITE: return "non-finite input";
    case KVQ_ERR_WORKSPACE: return "workspace missing or too small";
    case KVQ_ERR_LAUNCH: return "HIP runtime error";
    case KVQ_ERR_UNSUPPORTED: return "unsupported shape or format";
    case KVQ_ERR_DEVICE: return "device-side fault reported";
    default: return "unknown error";
  }
}

extern "C" int32_t kvq_workspace_bytes(int32_t fmt, const kvq_cache* kcache, const kvq_launch* l,
                                       int32_t ctx_len, int64_t* bytes) {
  if (!bytes) return KVQ_ERR_ARG;
  Plan plan;
  const int32_t rc = make_plan(fmt, kcache, l, ctx_len, &plan);
  if (rc) return rc;
  *bytes = plan.ws.total;
  return KVQ_OK;
}

extern "C" int32_t kvq_decode_attn(const void* q, const kvq_cache* kcache, const kvq_cache* vcache,
                                   int32_t fmt, int32_t ctx_len, float threshold, float* out,
                                   const kvq_launch* l) {
  if (!q || !kcache || !out || !l) return KVQ_ERR_ARG;
  if (!(threshold >= 0.0f) || !(threshold < 1.0f)) return KVQ_ERR_RANGE;   // also rejects NaN
  if (l->flags & ~int32_t(KVQ_LAUNCH_COOPERATIVE)) return KVQ_ERR_ARG;
  Plan plan;
  int32_t rc = make_plan(fmt, kcache, l, ctx_len, &plan);
  if (rc) return rc;
  if (!vcache) return KVQ_ERR_UNSUPPORTED;                 // latent caches: not in this kernel family
  if (vcache->batch != kcache->batch || vcache->heads != kcache->heads ||
      vcache->capacity != kcache->capacity || vcache->dim != 128)
    return KVQ_ERR_ARG;
  if (!kcache->codes || !kcache->scales || !vcache->codes || !vcache->scales) return KVQ_ERR_ARG;
  if (!aligned16(kcache->codes) || !aligned16(kcache->scales) || !aligned16(vcache->codes) ||
      !aligned16(vcache->scales) || !aligned16(q) || !aligned16(out) ||
      (l->mask_out && !aligned16(l->mask_out)) || (l->workspace && !aligned16(l->workspace)))
    return KVQ_ERR_ALIGN;
  if (!l->workspace || l->workspace_bytes < plan.ws.total) return KVQ_ERR_WORKSPACE;

  unsigned char* ws = static_cast<unsigned char*>(l->workspace);
  kvq::GqaArgs a{};
  a.q = q;
  a.kc = static_cast<const uint8_t*>(kcache->codes);
  a.ks = static_cast<const uint8_t*>(kcache->scales);
  a.vc = static_cast<const uint8_t*>(vcache->codes);
  a.vs = static_cast<const uint8_t*>(vcache->scales);
  a.out = out;
  a.mask_out = l->mask_out;
  a.hdr = reinterpret_cast<WsHeader*>(ws);
  a.kept_mass = reinterpret_cast<float*>(ws + plan.ws.kept_mass);
  a.bgstat = reinterpret_cast<unsigned long long*>(ws + plan.ws.bgstat);
  a.lse = reinterpret_cast<unsigned long long*>(ws + plan.ws.lse);
  a.split_ml = reinterpret_cast<unsigned long long*>(ws + plan.ws.split_ml);
  a.flags = reinterpret_cast<unsigned long long*>(ws + plan.ws.flags);
  a.pmass = reinterpret_cast<unsigned long long*>(ws + plan.ws.pmass);
  a.partial = reinterpret_cast<unsigned long long*>(ws + plan.ws.partial);
  a.B = kcache->batch;
  a.Hkv = kcache->heads;
  a.Hq = l->q_heads;
  a.ctx = ctx_len;
  a.cap = kcache->capacity;
  a.S = plan.S;
  a.P = plan.P;
  a.mask_words = (ctx_len + 31) / 32;
  a.q_bf16 = l->q_dtype == KVQ_Q_BF16;
  a.fmt = fmt;
  const float sigma = l->softmax_scale > 0.0f ? l->softmax_scale
                                             : static_cast<float>(1.0 / std::sqrt(static_cast<double>(kcache->dim)));
  a.sigma_log2e = static_cast<float>(static_cast<double>(sigma) * 1.4426950408889634);
  a.tau = threshold;
  a.times = reinterpret_cast<unsigned long long*>(l->phase_times);

  const void* kern = kvq::gqa_kernel(fmt, plan.G);
  if (!kern) return KVQ_ERR_UNSUPPORTED;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kvq::kThreads, plan.lds) != hipSuccess)
    return KVQ_ERR_LAUNCH;
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (int64_t(per_cu) * device_info(dev).cus < plan.nwg) return KVQ_ERR_UNSUPPORTED;
  void* args[] = {&a};
  const hipStream_t st = static_cast<hipStream_t>(l->stream);
  const hipError_t e =
      (l->flags & KVQ_LAUNCH_COOPERATIVE)
          ? hipLaunchCooperativeKernel(kern, dim3(plan.nwg), dim3(kvq::kThreads), args, unsigned(plan.lds), st)
          : hipLaunchKernel(kern, dim3(plan.nwg), dim3(kvq::kThreads), args, unsigned(plan.lds), st);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return KVQ_ERR_LAUNCH;
  }
  return KVQ_OK;
}

extern "C" int32_t kvq_phase_count(const kvq_launch* l, int32_t* workgroups, int32_t* stamps) {
  if (!l || !l->workspace || !workgroups || !stamps) return KVQ_ERR_ARG;
  if (hipStreamSynchronize(static_cast<hipStream_t>(l->stream)) != hipSuccess) return KVQ_ERR_LAUNCH;
  WsHeader h;
  if (hipMemcpy(&h, l->workspace, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess) return KVQ_ERR_LAUNCH;
  *workgroups = h.nwg;
  *stamps = kvq::kStamps;
  return KVQ_OK;
}

extern "C" int32_t kvq_stats(const kvq_launch* l, kvq_stats_t* out, float* kept_mass) {
  if (!l || !out || !l->workspace) return KVQ_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(l->stream);
  if (hipStreamSynchronize(st) != hipSuccess) return KVQ_ERR_LAUNCH;
  WsHeader h;
  if (hipMemcpy(&h, l->workspace, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess) return KVQ_ERR_LAUNCH;
  std::memset(out, 0, sizeof(*out));
  const int G = h.kv_heads > 0 ? h.q_heads / h.kv_heads : 0;
  int64_t cb = 0, sb = 0;
  if (h.batch > 0 && kvq_row_bytes(h.fmt, 128, &cb, &sb) == KVQ_OK) {
    out->positions = int64_t(h.batch) * h.kv_heads * h.ctx;
    out->pairs = int64_t(h.batch) * h.q_heads * h.ctx;
    out->k_bytes = out->positions * (cb + sb);
    out->v_bytes_dense = out->positions * (cb + sb);
  }
  (void)G;
  if (h.batch > 0) {
    const WsLayout w = kvq::ws_layout(h.batch, h.kv_heads, h.q_heads, h.splits, h.v_dim);
    const int64_t BG = int64_t(h.batch) * h.kv_heads;
    std::vector<unsigned long long> st(size_t(2 * BG));
    if (hipMemcpy(st.data(), static_cast<unsigned char*>(l->workspace) + w.bgstat, st.size() * 8,
                  hipMemcpyDeviceToHost) != hipSuccess)
      return KVQ_ERR_LAUNCH;
    for (int64_t i = 0; i < BG; ++i) {
      out->kept_pairs += int64_t(st[2 * i]);
      out->rows_fetched += int64_t(st[2 * i + 1]);
    }
    out->v_bytes = out->rows_fetched * (cb + sb);
  }
  out->status = int32_t(h.status);
  out->splits = h.splits;
  out->batch = h.batch;
  out->q_heads = h.q_heads;
  if (kept_mass && h.batch > 0) {
    const WsLayout w = kvq::ws_layout(h.batch, h.kv_heads, h.q_heads, h.splits, h.v_dim);
    if (hipMemcpy(kept_mass, static_cast<unsigned char*>(l->workspace) + w.kept_mass,
                  sizeof(float) * size_t(h.batch) * h.q_heads, hipMemcpyDeviceToHost) != hipSuccess)
      return KVQ_ERR_LAUNCH;
  }
  return h.status ? KVQ_ERR_DEVICE : KVQ_OK;
}
