// Internal types shared by the host entry points (kvq_api.cpp) and the HIP
// kernels. Not part of the public C ABI.
#pragma once

#include <stdint.h>

namespace kvq {

constexpr int kThreads = 1024;          // threads per workgroup (16 wave64s, one workgroup per CU)
constexpr int kWaves = kThreads / 64;
constexpr int kChunk = 64;              // positions per wave chunk (one ballot word)

// Device fault bits reported through WsHeader::status.
constexpr uint32_t kStatusWaitTimeout = 1u;   // a bounded wait gave up

// Retries of a bounded wait before it gives up (each retry sleeps briefly and
// re-reads: about half a second in all), and the short limit of the test aid
// that withholds one split's statistics.
constexpr uint32_t kSpinLimit = 1u << 23;
constexpr uint32_t kTestSpinLimit = 1u << 12;

// Workspace header. The first 256 bytes of every workspace; the rest holds the
// per-split statistics and partial outputs of the last call.
struct WsHeader {
  uint32_t epoch;                       // tag of the last call (0 in a fresh workspace)
  uint32_t groups_done;                 // groups past their LSE exchange in the running call (returns to 0)
  uint32_t status;                      // sticky device fault bits
  uint32_t launches;                    // kernel launches of the last call (the grouped plans may need several)
  long long live_off;                   // byte offset of the per-workgroup live-tile counts (int32 [nwg])
  long long kdrop_off;                  // byte offset of the per-workgroup dropped key positions (int32 [nwg]; 0: none)
  int32_t batch, q_heads, kv_heads, ctx;
  int32_t splits, positions_per_split, fmt, v_dim;
  int32_t nwg, k_row_bytes;
  int32_t v_row_bytes, pad2;
  uint8_t pad1[256 - 16 - 16 - 32 - 16];
};
static_assert(sizeof(WsHeader) == 256, "header is one 256-byte line");

// Byte offsets of the workspace regions for one call's plan. Every value
// that one workgroup hands to another is a 64-bit "tagged word": the call's
// epoch in the high half, the 32-bit payload in the low half. A reader polls
// until the tag matches, so no fence or counter orders the hand-off.
struct WsLayout {
  int64_t kept_mass;   // float [B*Hq]
  int64_t bgstat;      // u64 [B*Hkv][2]: kept pairs, value rows fetched
  int64_t lse;         // tagged [B*Hkv][G]: log2-domain log-sum-exp per head
  int64_t split_ml;    // tagged [B*Hkv][S][G][2]: per-split (max, sum) in the log2 domain
  int64_t flags;       // tagged [B*Hkv][S]: rows fetched << 18 | kept pairs of the split
  int64_t act;         // tagged [B*Hkv][S]: 1 if the split publishes a partial output (it keeps a row)
  int64_t pmass;       // tagged [B*Hkv][S][G]: per-split kept mass
  int64_t partial;     // tagged [B*Hkv][S][G][Dv]: per-split partial outputs
  int64_t live;        // int32 [B*Hkv][S]: 64-position chunks of the split holding a kept row
  int64_t pre_ml;      // tagged [B*Hkv][S][G][2]: key skipping, (max, sum) over the split's candidate blocks
  int64_t kdrop;       // int32 [B*Hkv][S]: key skipping, key positions the split left out
  int64_t total;
};

inline int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

inline WsLayout ws_layout(int B, int Hkv, int Hq, int S, int Dv) {
  const int G = Hq / Hkv;
  const int64_t BG = int64_t(B) * Hkv;
  WsLayout w;
  int64_t off = 256;
  w.kept_mass = off; off = align256(off + int64_t(B) * Hq * 4);
  w.bgstat = off;    off = align256(off + BG * 16);
  w.lse = off;       off = align256(off + BG * G * 8);
  w.split_ml = off;  off = align256(off + BG * S * G * 16);
  w.flags = off;     off = align256(off + BG * S * 8);
  w.act = off;       off = align256(off + BG * S * 8);
  w.pmass = off;     off = align256(off + BG * S * G * 8);
  w.partial = off;   off = align256(off + BG * S * G * int64_t(Dv) * 8);
  w.live = off;      off = align256(off + BG * S * 4);
  w.pre_ml = off;    off = align256(off + BG * S * G * 16);
  w.kdrop = off;     off = align256(off + BG * S * 4);
  w.total = off;
  return w;
}

// Arguments of the fused grouped-query kernel (one struct, passed by value).
struct GqaArgs {
  const void* q;                  // [B][Hq][D] float32 or bfloat16
  const uint8_t* kc;              // key code plane
  const uint8_t* ks;              // key scale plane
  const uint8_t* vc;              // value code plane
  const uint8_t* vs;              // value scale plane
  float* out;                     // [B][Hq][D]
  uint32_t* mask_out;             // optional keep bits
  WsHeader* hdr;
  float* kept_mass;
  unsigned long long* bgstat;
  unsigned long long* lse;        // tagged
  unsigned long long* split_ml;   // tagged
  unsigned long long* flags;      // tagged
  unsigned long long* act;        // tagged
  unsigned long long* pmass;      // tagged
  unsigned long long* partial;    // tagged
  int32_t B, Hkv, Hq, ctx, cap;
  int32_t S, P;                   // splits per (b, kv head), positions per split (multiple of 64)
  int32_t mask_words;             // ceil(ctx / 32)
  int32_t q_bf16;
  int32_t fmt;
  float sigma_log2e;              // softmax scale times log2(e)
  float tau;                      // threshold on the normalized weight
  unsigned long long* times;      // optional [nwg][16] phase stamps
  uint32_t spin_limit;            // retries of a bounded wait
  int32_t withhold;               // test aid: split 0 of group 0 does not publish its statistics
  int32_t* live;                  // [nwg] live 64-position chunks per workgroup
  long long live_off;             // its byte offset in the workspace (recorded in the header)
  int32_t bg0, ngroups;           // this launch covers groups bg0 .. bg0 + ngroups - 1 (of B * Hkv)
  int32_t launches;               // launches of the call
  // key skipping (kskip != 0): block summaries [B*Hkv][knorm_pitch] (largest key
  // norm per 64 rows), the candidates' statistics, dropped positions per
  // workgroup and the optional dropped-block map [B*Hkv][ceil(ctx/64)]
  int32_t kskip;
  int32_t knorm_pitch;
  const float* knorm;
  unsigned long long* pre_ml;     // tagged
  int32_t* kdrop;
  long long kdrop_off;
  uint8_t* kskip_out;
};

// Arguments of the two MLA kernels.
struct MlaArgs {
  const void* q;                  // [B][H][576] bfloat16
  const uint8_t* kc;              // latent code plane [B][cap][576] (e4m3)
  const uint8_t* ks;              // latent scale plane [B][cap][5] (fp32)
  float* out;                     // [B][H][512]
  WsHeader* hdr;
  float* kept_mass;               // [B][H]
  unsigned long long* bgstat;     // [B][2]
  unsigned long long* split_ml;   // tagged [B][S][H][2]
  int32_t* kcount;                // [B][S] kept rows published by each split
  int32_t* kpairs;                // [B][S] kept (head, position) pairs per split
  int32_t* kpos;                  // [B][S][P] positions of kept rows
  float* kp;                      // [B][S][P][H] weights of kept rows (0 where a head skips)
  float* opart;                   // [B][H/32][4][R][32][128] output partials of row ranges
  float* mpart;                   // [B][H/32][R][32] kept-mass partials of row ranges
  uint32_t* ocnt;                 // [B][H/32][4] row ranges finished (0 between calls)
  unsigned long long* done;       // tagged [B][H/64][R]: every-row-kept ranges that wrote their partials
  int32_t R;                      // row ranges launched (per output block, or per sequence at threshold 0)
  int32_t tpe;                    // 32-position tiles per tile-maximum entry of the scores kernel (1 or 2)
  int32_t scores_out;             // 1: kp holds every row's log2-domain scores (threshold 0, mla_out_dense)
  float* lseo;                    // [B][H] log2-domain LSE per head (written when scores_out)
  unsigned long long* lsep;       // tagged [B][H]: log2-domain LSE per head, published by the scores kernel
  uint32_t* mask_out;             // optional keep bits [B][H][mask_words]
  int32_t mask_words;             // ceil(ctx / 32)
  int32_t B, Hq, ctx, cap;
  int32_t S, P;
  float sigma_log2e;
  float tau;
  unsigned long long* times;      // optional [nwg][16] phase stamps of mla_scores
  uint32_t spin_limit;            // retries of a bounded wait
  int32_t withhold;               // test aid: split 0 of sequence 0 does not publish its statistics
  int32_t* live;                  // [B][S] 32-position tiles each scores workgroup re-scored
  long long live_off;             // its byte offset in the workspace (recorded in the header)
};

struct MlaLayout {
  int64_t kept_mass, bgstat, split_ml, kcount, kpairs, kpos, kp, opart, mpart, ocnt, done, lseo, lsep, live, total;
};

// The first two regions match ws_layout() so kvq_stats reads both families
// alike. The range counters (which must hold 0 between calls) and the done
// words come next, sized for the most ranges a plan uses, so their offsets
// depend on the batch and head count only: calls with different context
// lengths on one workspace find them where the previous call left them.
// SP: positions published per sequence over all splits (S * P).
constexpr int kMaxRanges = 64;
inline MlaLayout mla_ws_layout(int B, int H, int S, int64_t SP, int R) {
  MlaLayout w;
  int64_t off = 256;
  w.kept_mass = off; off = align256(off + int64_t(B) * H * 4);
  w.bgstat = off;    off = align256(off + int64_t(B) * 16);
  w.ocnt = off;      off = align256(off + int64_t(B) * (H / 32) * 4 * 4);
  w.done = off;      off = align256(off + int64_t(B) * (H >= 64 ? H / 64 : 1) * kMaxRanges * 8);
  w.lseo = off;      off = align256(off + int64_t(B) * H * 4);
  w.lsep = off;      off = align256(off + int64_t(B) * H * 8);
  w.split_ml = off;  off = align256(off + int64_t(B) * S * H * 16);
  w.kcount = off;    off = align256(off + int64_t(B) * S * 4);
  w.kpairs = off;    off = align256(off + int64_t(B) * S * 4);
  w.kpos = off;      off = align256(off + int64_t(B) * SP * 4);
  w.kp = off;        off = align256(off + int64_t(B) * SP * int64_t(H) * 4);
  w.opart = off;     off = align256(off + int64_t(B) * (H / 32) * 4 * R * 32 * 128 * 4);
  w.mpart = off;     off = align256(off + int64_t(B) * (H / 32) * R * 32 * 4);
  w.live = off;      off = align256(off + int64_t(B) * S * 4);
  w.total = off;
  return w;
}

constexpr int kStamps = 10;       // phase stamps per workgroup (7..9 split the V pass)

// Latent output contraction at threshold 0: mla_out's per-block row ranges
// hold at least kOutMinRows rows (the rest of the launched ranges exit at once).
constexpr int kOutMinRows = 2048;
constexpr int kDenseOutThreads = 512;       // workgroup size of the latent output kernel at threshold 0

// Floats of the first LDS region of the grouped kernel: scores [G][P], the
// cross-wave reduction [kWaves][G][128], and the merge's slice partials
// [E][S] (E = ceil(G*128 / S)), kept-mass inputs [nh][S] (nh = heads a
// workgroup sums: 1 if S >= G, else ceil(G / S)) and flags [S].
// Output elements each workgroup of a group sums in the merge: ceil(G*128/S)
// rounded up to even, so every slice starts on a 16-byte boundary.
inline __host__ __device__ int gqa_merge_slice(int G, int S) { return 2 * ((G * 128 + 2 * S - 1) / (2 * S)); }

inline __host__ __device__ int gqa_sc_floats(int G, int P, int S) {
  int n = G * P;
  if (kWaves * G * 128 > n) n = kWaves * G * 128;
  const int E = gqa_merge_slice(G, S);
  const int nh = S >= G ? 1 : (G + S - 1) / S;
  const int m = S * (1 + E + nh);
  if (m > n) n = m;
  return (n + 3) & ~3;                  // keeps the regions after it 16-byte aligned
}
constexpr int kMlaStamps = 5;     // latent path: start, scores start, scores end, lse known, lists published

}  // namespace kvq
