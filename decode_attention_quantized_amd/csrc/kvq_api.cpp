// Host entry points of the decode-attention C ABI (see include/kvq.h):
// argument validation, the split plan, workspace layout, the cooperative
// launch and the statistics readback. The kernels live in kvq_gqa.hip.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <algorithm>
#include <mutex>
#include <vector>

#include "kvq.h"
#include "kvq_internal.h"

namespace kvq {
size_t gqa_lds_bytes(int fmt, int G, int P, int S);
const void* gqa_kernel(int fmt, int G, int mode);   // mode 0: exact rule, 1: single-pass rule, 2: key skipping
size_t mla_lds_bytes(int H, int P, int S, int tpe);
const void* mla_scores_kernel(int H);
const void* mla_out_kernel();
size_t mla_out_dense_lds(int H);
const void* mla_out_dense_kernel(int H);
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
  bool mla = false;
  int S = 0, P = 0, G = 0, Dv = 0;
  size_t lds = 0;
  int nwg = 0;
  int threads = 0;
  int R = 1;                                              // latent output: row ranges per block
  int tpe = 2;                                            // latent scores: 32-position tiles per tile maximum
  int gpl = 0, nsub = 1;                                  // grouped plans: groups per launch, launches
  WsLayout ws{};
  kvq::MlaLayout mws{};
  int64_t total = 0;
};

bool is_gqa_fmt(int fmt) {
  return fmt == KVQ_Q8_0 || fmt == KVQ_Q4_0 || fmt == KVQ_LUT3 || fmt == KVQ_LUT3_WHT;
}

// MLA shape: H query heads over one 576-wide fp8 latent per sequence, values =
// the first 512 dims, bf16 queries. One 4-wave workgroup per CU by default.
int32_t make_mla_plan(const kvq_cache* k, const kvq_launch* l, int32_t ctx_len, Plan* plan) {
  if (k->heads != 1 || k->dim != 576) return KVQ_ERR_UNSUPPORTED;
  if (l->v_dim != 512) return KVQ_ERR_UNSUPPORTED;
  if (l->q_dtype != KVQ_Q_BF16) return KVQ_ERR_UNSUPPORTED;
  const int H = l->q_heads;
  if (H != 32 && H != 64 && H != 128) return KVQ_ERR_UNSUPPORTED;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return KVQ_ERR_LAUNCH;
  const DeviceInfo di = device_info(dev);
  if (di.cus <= 0) return KVQ_ERR_LAUNCH;
  int S;
  if (l->splits > 0) {
    S = l->splits;
  } else {
    int64_t s = di.cus / k->batch;
    if (s < 1) s = 1;
    const int64_t most = (ctx_len + 63) / 64;
    if (s > most) s = most;
    S = int(s);
  }
  int P = (ctx_len + S - 1) / S;
  P = (P + 63) / 64 * 64;
  S = (ctx_len + P - 1) / P;
  if (S > 1024) return KVQ_ERR_UNSUPPORTED;
  // one tile maximum per 32-position tile when the table fits, else one per 64
  int tpe = 1;
  size_t lds = kvq::mla_lds_bytes(H, P, S, 1);
  if (lds > size_t(di.max_lds)) {
    tpe = 2;
    lds = kvq::mla_lds_bytes(H, P, S, 2);
  }
  if (lds > size_t(di.max_lds)) return KVQ_ERR_UNSUPPORTED;
  plan->tpe = tpe;
  plan->mla = true;
  plan->S = S;
  plan->P = P;
  plan->G = H;
  plan->Dv = 512;
  plan->lds = lds;
  plan->nwg = k->batch * S;
  plan->threads = 4 * H;                                 // two waves per 32-head block
  // row ranges of the every-row-kept output: one workgroup per CU over the
  // batch and its 64-head sets, at least 64 rows each
  plan->R = int(std::max<int64_t>(1, std::min<int64_t>({kvq::kMaxRanges,
                                                          di.cus / (int64_t(k->batch) * std::max(1, H / 64)),
                                                          (ctx_len + 63) / 64})));
  plan->mws = kvq::mla_ws_layout(k->batch, H, S, int64_t(S) * P, plan->R);
  plan->total = plan->mws.total;
  return KVQ_OK;
}

// Validate shapes shared by every entry point and pick splits.
int32_t make_plan(int32_t fmt, const kvq_cache* k, const kvq_launch* l, int32_t ctx_len, Plan* plan) {
  if (!k || !l || !plan) return KVQ_ERR_ARG;
  if (fmt < KVQ_Q8_0 || fmt > KVQ_LUT3_WHT) return KVQ_ERR_ARG;
  if (k->batch <= 0 || k->heads <= 0 || k->dim <= 0 || k->capacity <= 0) return KVQ_ERR_ARG;
  if (l->q_heads <= 0 || l->q_heads % k->heads) return KVQ_ERR_ARG;
  if (l->q_dtype != KVQ_Q_F32 && l->q_dtype != KVQ_Q_BF16) return KVQ_ERR_ARG;
  if (ctx_len < 1 || ctx_len > k->capacity) return KVQ_ERR_RANGE;
  if (fmt == KVQ_FP8_B128) return make_mla_plan(k, l, ctx_len, plan);
  if (!is_gqa_fmt(fmt)) return KVQ_ERR_UNSUPPORTED;
  if (k->dim != 128) return KVQ_ERR_UNSUPPORTED;
  const int G = l->q_heads / k->heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return KVQ_ERR_UNSUPPORTED;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return KVQ_ERR_LAUNCH;
  const DeviceInfo di = device_info(dev);
  if (di.cus <= 0) return KVQ_ERR_LAUNCH;

  const int64_t BG = int64_t(k->batch) * k->heads;
  // All workgroups of a launch must be resident (one per CU) and a split's
  // scores must fit in LDS. A call whose groups (sequence, kv head) do not
  // fit one launch under both limits runs in several launches on the stream,
  // each over an equal share of the groups with the splits refilling the CUs
  // (fewer groups per launch: more splits, fewer positions per split).
  int S = 0, P = 0;
  int64_t gpl = BG;                                       // groups per launch
  size_t lds = 0;
  for (int64_t nsub = 1;; ++nsub) {
    gpl = (BG + nsub - 1) / nsub;
    if (nsub > 1 && (BG + gpl - 1) / gpl < nsub) continue;   // same share as a smaller count
    if (l->splits > 0) {
      S = l->splits;
    } else {
      int64_t s = di.cus / gpl;
      if (s < 1) s = 1;
      const int64_t most = (ctx_len + kvq::kChunk - 1) / kvq::kChunk;
      if (s > most) s = most;
      S = int(s);
    }
    P = (ctx_len + S - 1) / S;
    P = (P + kvq::kChunk - 1) / kvq::kChunk * kvq::kChunk;
    S = (ctx_len + P - 1) / P;                           // drop splits that would be empty
    // P <= 8192: per-split counts are packed in 14/18 bits; the in-kernel
    // exchanges read at most two of the group's split statistics, one
    // 16-byte piece of partial outputs and two kept-mass and flag words per
    // thread
    const int64_t E = kvq::gqa_merge_slice(G, S);
    const int64_t nh = S >= G ? 1 : (G + S - 1) / S;
    const bool fits = P <= 8192 && S <= 2048 && BG * S <= (int64_t(1) << 30) && gpl * S <= di.cus &&
                      int64_t(S) * G <= 2 * kvq::kThreads && (E / 2) * S <= kvq::kThreads &&
                      nh * S <= 2 * kvq::kThreads;
    lds = fits ? kvq::gqa_lds_bytes(fmt, G, P, S) : 0;
    if (fits && lds <= size_t(di.max_lds)) break;
    if (gpl == 1) return KVQ_ERR_UNSUPPORTED;               // one group alone does not fit
  }

  plan->S = S;
  plan->P = P;
  plan->G = G;
  plan->Dv = 128;
  plan->lds = lds;
  plan->gpl = int(gpl);
  plan->nsub = int((BG + gpl - 1) / gpl);
  plan->nwg = int(gpl * S);                               // workgroups of a (full) launch
  plan->threads = kvq::kThreads;
  plan->ws = kvq::ws_layout(k->batch, k->heads, l->q_heads, S, plan->Dv);
  plan->total = plan->ws.total;
  return KVQ_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

float sigma_log2e_of(const kvq_launch* l, int dim_qk) {
  const float sigma = l->softmax_scale > 0.0f ? l->softmax_scale
                                             : static_cast<float>(1.0 / std::sqrt(static_cast<double>(dim_qk)));
  return static_cast<float>(static_cast<double>(sigma) * 1.4426950408889634);
}

hipError_t launch(const void* kern, int grid, int threads, void* arg, size_t lds, const kvq_launch* l) {
  void* args[] = {arg};
  const hipStream_t st = static_cast<hipStream_t>(l->stream);
  return (l->flags & KVQ_LAUNCH_COOPERATIVE)
             ? hipLaunchCooperativeKernel(kern, dim3(grid), dim3(threads), args, unsigned(lds), st)
             : hipLaunchKernel(kern, dim3(grid), dim3(threads), args, unsigned(lds), st);
}

int32_t launch_mla(const void* q, const kvq_cache* kcache, const kvq_cache* vcache, int32_t ctx_len,
                   float threshold, float* out, const kvq_launch* l, const Plan& plan) {
  if (vcache) return KVQ_ERR_ARG;                         // the values are the latent's first 512 dims
  if (!kcache->codes || !kcache->scales) return KVQ_ERR_ARG;
  if (!aligned16(kcache->codes) || !aligned16(kcache->scales) || !aligned16(q) || !aligned16(out) ||
      (l->workspace && !aligned16(l->workspace)))
    return KVQ_ERR_ALIGN;
  if (l->mask_out && !aligned16(l->mask_out)) return KVQ_ERR_ALIGN;
  if (!l->workspace || l->workspace_bytes < plan.total) return KVQ_ERR_WORKSPACE;
  unsigned char* ws = static_cast<unsigned char*>(l->workspace);
  kvq::MlaArgs a{};
  a.q = q;
  a.kc = static_cast<const uint8_t*>(kcache->codes);
  a.ks = static_cast<const uint8_t*>(kcache->scales);
  a.out = out;
  a.hdr = reinterpret_cast<WsHeader*>(ws);
  a.kept_mass = reinterpret_cast<float*>(ws + plan.mws.kept_mass);
  a.bgstat = reinterpret_cast<unsigned long long*>(ws + plan.mws.bgstat);
  a.split_ml = reinterpret_cast<unsigned long long*>(ws + plan.mws.split_ml);
  a.kcount = reinterpret_cast<int32_t*>(ws + plan.mws.kcount);
  a.kpairs = reinterpret_cast<int32_t*>(ws + plan.mws.kpairs);
  a.kpos = reinterpret_cast<int32_t*>(ws + plan.mws.kpos);
  a.kp = reinterpret_cast<float*>(ws + plan.mws.kp);
  a.opart = reinterpret_cast<float*>(ws + plan.mws.opart);
  a.mpart = reinterpret_cast<float*>(ws + plan.mws.mpart);
  a.ocnt = reinterpret_cast<uint32_t*>(ws + plan.mws.ocnt);
  a.done = reinterpret_cast<unsigned long long*>(ws + plan.mws.done);
  a.lseo = reinterpret_cast<float*>(ws + plan.mws.lseo);
  a.lsep = reinterpret_cast<unsigned long long*>(ws + plan.mws.lsep);
  a.live = reinterpret_cast<int32_t*>(ws + plan.mws.live);
  a.live_off = plan.mws.live;
  a.mask_out = l->mask_out;
  a.mask_words = (ctx_len + 31) / 32;
  // threshold 0 keeps every row: the output contraction is split over row
  // ranges (mla_out_dense when all its workgroups fit on the GPU at once,
  // else mla_out's per-block ranges); a positive threshold keeps few rows,
  // one range per mla_out block
  a.R = threshold == 0.0f ? plan.R : 1;
  a.tpe = plan.tpe;
  a.B = kcache->batch;
  a.Hq = l->q_heads;
  a.ctx = ctx_len;
  a.cap = kcache->capacity;
  a.S = plan.S;
  a.P = plan.P;
  a.sigma_log2e = sigma_log2e_of(l, 192);                 // default scale 1/sqrt(qk_nope + rope = 192)
  a.tau = threshold;
  a.times = reinterpret_cast<unsigned long long*>(l->phase_times);
  a.withhold = (l->flags & KVQ_TEST_WITHHOLD) != 0;
  a.spin_limit = a.withhold ? kvq::kTestSpinLimit : kvq::kSpinLimit;
  const void* ks = kvq::mla_scores_kernel(plan.G);
  if (!ks) return KVQ_ERR_UNSUPPORTED;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, ks, plan.threads, plan.lds) != hipSuccess)
    return KVQ_ERR_LAUNCH;
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (int64_t(per_cu) * device_info(dev).cus < plan.nwg) return KVQ_ERR_UNSUPPORTED;
  // threshold 0 with mla_out_dense (all its workgroups resident at once): the
  // scores kernel stores every score in its first pass and skips the re-score
  // pass; the output kernel turns scores into weights with the LSE
  const void* kd = threshold == 0.0f ? kvq::mla_out_dense_kernel(plan.G) : nullptr;
  const size_t dl = kvq::mla_out_dense_lds(plan.G);
  bool dense = false;
  if (kd && dl <= size_t(device_info(dev).max_lds)) {
    int pd = 0;
    dense = hipOccupancyMaxActiveBlocksPerMultiprocessor(&pd, kd, kvq::kDenseOutThreads, dl) == hipSuccess &&
            int64_t(pd) * device_info(dev).cus >= int64_t(kcache->batch) * (plan.G / 64) * a.R;
  }
  a.scores_out = dense ? 1 : 0;
  hipError_t e = launch(ks, plan.nwg, plan.threads, &a, plan.lds, l);
  if (e == hipSuccess) {
    if (dense) e = launch(kd, kcache->batch * (plan.G / 64) * a.R, kvq::kDenseOutThreads, &a, dl, l);
    else e = launch(kvq::mla_out_kernel(), kcache->batch * (plan.G / 32) * 4 * a.R, 256, &a, 0, l);
  }
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return KVQ_ERR_LAUNCH;
  }
  return KVQ_OK;
}

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
  // Size for every context length up to ctx_len: rounding P up to whole
  // 64-position chunks makes the split count of a plan fall and rise again
  // as the context grows (4096 positions over 64 splits of 64, 4097 over 33
  // of 128), so a decode loop's later, shorter or longer, calls may need more
  // than the plan of ctx_len. Every plan for ctx' <= ctx_len has
  //   S' <= s0 = the requested splits, else min(CUs / sequences, ceil(ctx_len / 64)),
  //   S' * P' < ctx' + P' <= ctx_len + ceil(ctx_len / s_cap) + 126,
  //   R' <= R of ctx_len,
  // and every region of a layout grows with these.
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return KVQ_ERR_LAUNCH;
  const int64_t cus = device_info(dev).cus;
  const int64_t chunks = (int64_t(ctx_len) + 63) / 64;
  if (plan.mla) {
    const int64_t cap = l->splits > 0 ? l->splits : std::max<int64_t>(1, cus / kcache->batch);
    const int64_t s_up = std::min(cap, chunks);
    const int64_t sp_up = int64_t(ctx_len) + (int64_t(ctx_len) + cap - 1) / cap + 126;
    const kvq::MlaLayout w = kvq::mla_ws_layout(kcache->batch, plan.G, int(s_up), sp_up, plan.R);
    *bytes = std::max(plan.total, w.total);
  } else {
    // a shorter context needs at most as many launches, so at least as many
    // groups per launch and at most as many splits
    const int64_t s_up = l->splits > 0 ? l->splits : std::min(std::max<int64_t>(1, cus / plan.gpl), chunks);
    const kvq::WsLayout w = kvq::ws_layout(kcache->batch, kcache->heads, l->q_heads, int(s_up), plan.Dv);
    *bytes = std::max(plan.total, w.total);
  }
  return KVQ_OK;
}

extern "C" int32_t kvq_decode_attn(const void* q, const kvq_cache* kcache, const kvq_cache* vcache,
                                   int32_t fmt, int32_t ctx_len, float threshold, float* out,
                                   const kvq_launch* l) {
  if (!q || !kcache || !out || !l) return KVQ_ERR_ARG;
  if (!(threshold >= 0.0f) || !(threshold < 1.0f)) return KVQ_ERR_RANGE;   // also rejects NaN
  if (l->flags & ~int32_t(KVQ_LAUNCH_COOPERATIVE | KVQ_SKIP_RUNNING | KVQ_TEST_WITHHOLD | KVQ_SKIP_KEYS))
    return KVQ_ERR_ARG;
  const bool kskip = (l->flags & KVQ_SKIP_KEYS) != 0;
  if (kskip && (l->flags & KVQ_SKIP_RUNNING)) return KVQ_ERR_UNSUPPORTED;   // one skip rule per call
  Plan plan;
  int32_t rc = make_plan(fmt, kcache, l, ctx_len, &plan);
  if (rc) return rc;
  if (plan.mla) {
    if (l->flags & (KVQ_SKIP_RUNNING | KVQ_SKIP_KEYS)) return KVQ_ERR_UNSUPPORTED;   // latent kernels: exact rule only
    return launch_mla(q, kcache, vcache, ctx_len, threshold, out, l, plan);
  }
  if (!vcache) return KVQ_ERR_UNSUPPORTED;                 // latent caches: not in this kernel family
  if (vcache->batch != kcache->batch || vcache->heads != kcache->heads ||
      vcache->capacity != kcache->capacity || vcache->dim != 128)
    return KVQ_ERR_ARG;
  if (!kcache->codes || !kcache->scales || !vcache->codes || !vcache->scales) return KVQ_ERR_ARG;
  if (!aligned16(kcache->codes) || !aligned16(kcache->scales) || !aligned16(vcache->codes) ||
      !aligned16(vcache->scales) || !aligned16(q) || !aligned16(out) ||
      (l->mask_out && !aligned16(l->mask_out)) || (l->workspace && !aligned16(l->workspace)))
    return KVQ_ERR_ALIGN;
  if (kskip && !kcache->block_norms) return KVQ_ERR_ARG;
  if (kskip && (reinterpret_cast<uintptr_t>(kcache->block_norms) & 3)) return KVQ_ERR_ALIGN;
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
  a.act = reinterpret_cast<unsigned long long*>(ws + plan.ws.act);
  a.pmass = reinterpret_cast<unsigned long long*>(ws + plan.ws.pmass);
  a.partial = reinterpret_cast<unsigned long long*>(ws + plan.ws.partial);
  a.live = reinterpret_cast<int32_t*>(ws + plan.ws.live);
  a.live_off = plan.ws.live;
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
  a.sigma_log2e = sigma_log2e_of(l, kcache->dim);
  a.tau = threshold;
  a.times = reinterpret_cast<unsigned long long*>(l->phase_times);
  a.withhold = (l->flags & KVQ_TEST_WITHHOLD) != 0;
  a.spin_limit = a.withhold ? kvq::kTestSpinLimit : kvq::kSpinLimit;
  a.kskip = kskip;
  a.knorm = kcache->block_norms;
  a.knorm_pitch = (kcache->capacity + 63) / 64;
  a.pre_ml = reinterpret_cast<unsigned long long*>(ws + plan.ws.pre_ml);
  a.kdrop = reinterpret_cast<int32_t*>(ws + plan.ws.kdrop);
  a.kdrop_off = plan.ws.kdrop;
  a.kskip_out = l->key_skip_out;

  const void* kern = kvq::gqa_kernel(fmt, plan.G, kskip ? 2 : (l->flags & KVQ_SKIP_RUNNING) ? 1 : 0);
  if (!kern) return KVQ_ERR_UNSUPPORTED;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kvq::kThreads, plan.lds) != hipSuccess)
    return KVQ_ERR_LAUNCH;
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (int64_t(per_cu) * device_info(dev).cus < plan.nwg) return KVQ_ERR_UNSUPPORTED;
  // one launch per share of the groups, in order on the caller's stream
  // (each finishes before the next starts and advances the epoch)
  const int BG = kcache->batch * kcache->heads;
  a.launches = plan.nsub;
  for (int bg0 = 0; bg0 < BG; bg0 += plan.gpl) {
    a.bg0 = bg0;
    a.ngroups = std::min(plan.gpl, BG - bg0);
    const hipError_t e = launch(kern, a.ngroups * plan.S, kvq::kThreads, &a, plan.lds, l);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return KVQ_ERR_LAUNCH;
    }
  }
  return KVQ_OK;
}

extern "C" int32_t kvq_phase_count(const kvq_launch* l, int32_t* workgroups, int32_t* stamps) {
  if (!l || !l->workspace || !workgroups || !stamps) return KVQ_ERR_ARG;
  if (hipStreamSynchronize(static_cast<hipStream_t>(l->stream)) != hipSuccess) return KVQ_ERR_LAUNCH;
  WsHeader h;
  if (hipMemcpy(&h, l->workspace, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess) return KVQ_ERR_LAUNCH;
  *workgroups = h.nwg;
  *stamps = h.fmt == KVQ_FP8_B128 ? kvq::kMlaStamps : kvq::kStamps;
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
  if (h.batch > 0) {
    out->positions = int64_t(h.batch) * h.kv_heads * h.ctx;
    out->pairs = int64_t(h.batch) * h.q_heads * h.ctx;
    out->k_bytes = out->positions * h.k_row_bytes;
    out->v_bytes_dense = out->positions * h.v_row_bytes;
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
    out->v_bytes = out->rows_fetched * h.v_row_bytes;
  }
  if (h.batch > 0 && h.nwg > 0 && h.live_off > 0) {
    std::vector<int32_t> lv(size_t(h.nwg));
    if (hipMemcpy(lv.data(), static_cast<unsigned char*>(l->workspace) + h.live_off, lv.size() * 4,
                  hipMemcpyDeviceToHost) != hipSuccess)
      return KVQ_ERR_LAUNCH;
    for (int32_t v : lv) out->live_tiles += v;
  }
  if (h.batch > 0 && h.nwg > 0 && h.kdrop_off > 0) {
    std::vector<int32_t> kd(size_t(h.nwg));
    if (hipMemcpy(kd.data(), static_cast<unsigned char*>(l->workspace) + h.kdrop_off, kd.size() * 4,
                  hipMemcpyDeviceToHost) != hipSuccess)
      return KVQ_ERR_LAUNCH;
    for (int32_t v : kd) out->key_rows_skipped += v;
  }
  out->status = int32_t(h.status);
  out->launches = int32_t(h.launches);
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

// ---------------------------------------------------------------- no-allocation entry point
// A fixed device array stands in for the caller's workspace. Each GPU holds
// its own copy (zero at load, which is the state a fresh workspace must
// have; the kernels keep it valid from call to call). Host code never uses
// the array's name as an address: the device address of this device's copy
// comes from hipGetSymbolAddress, once per device, and is kept.
namespace {

constexpr int64_t kScratchBytes = int64_t(8) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

void* scratch_address(int dev) {
  static std::mutex mu;
  static void* addr[64] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (dev < 0 || dev >= 64) return nullptr;
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    addr[dev] = p;
  }
  return addr[dev];
}

}  // namespace

extern "C" int32_t kvq_decode_attn_noalloc(const void* q, const kvq_cache* kcache, const kvq_cache* vcache,
                                           int32_t fmt, int32_t ctx_len, float threshold, float* out,
                                           const kvq_launch* l) {
  if (!q || !kcache || !out || !l) return KVQ_ERR_ARG;
  Plan plan;
  const int32_t rc = make_plan(fmt, kcache, l, ctx_len, &plan);
  if (rc) return rc;
  if (plan.mla) return KVQ_ERR_UNSUPPORTED;              // the latent plans need far more than the array
  if (plan.total > kScratchBytes) return KVQ_ERR_WORKSPACE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return KVQ_ERR_LAUNCH;
  void* ws = scratch_address(dev);
  if (!ws) return KVQ_ERR_LAUNCH;
  kvq_launch lw = *l;
  lw.workspace = ws;
  lw.workspace_bytes = kScratchBytes;
  return kvq_decode_attn(q, kcache, vcache, fmt, ctx_len, threshold, out, &lw);
}
