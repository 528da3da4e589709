/*
 * kvq — single-token decode attention over a block-quantized KV cache, with
 * the sparse-V skip, for AMD Instinct MI355X (gfx950).
 *
 * Sources for what is computed (cited by page title and section):
 *  [SV]  "Пропуск 90% работы по деквантизации ускорил декодирование LLM на
 *        22,8%" (tproger.ru news item on sparse V dequantization):
 *        "Решение — не ускорять, а пропускать" — the softmax weights come from
 *        K before any V work, and a position whose attention weight is below
 *        1e-6 has its V dequantization *and* accumulation skipped entirely;
 *        "Почему это работает для любой квантизации" — the rule is format
 *        independent (q8_0, q4_0, turbo3 with a LUT codebook and a norm);
 *        FAQ — every K must still be dequantized to know the weights.
 *  [MLA] "FP8 MLA KV compression projection" (kernelindex.com), workload
 *        parameters: a 576-wide latent (kv_lora_rank 512 + qk_rope_head_dim
 *        64), fp8 with BlockWise1x128 scaling, 128 heads, qk_nope_head_dim 128.
 *
 * Conventions for every entry point:
 *  - Return 0 (KVQ_OK) on success or a negative KVQ_ERR_* code. All argument
 *    checks happen before any device work; a failed check launches nothing.
 *  - "host" pointers are ordinary CPU memory; "device" pointers are GPU memory
 *    (e.g. from hipMalloc or a torch CUDA tensor's data_ptr()).
 *  - The library allocates no device memory and keeps no global mutable state
 *    apart from a per-device cache of the compute-unit count. Calls that share
 *    a workspace must be serialized (same stream or explicit ordering).
 *  - kvq_decode_attn's workgroups hand data to one another inside a launch,
 *    so all of them must be resident at once: the plan launches at most one
 *    per compute unit, which holds when nothing else occupies the GPU's
 *    compute units (other kernels on concurrent streams included). When that
 *    cannot be ensured, KVQ_LAUNCH_COOPERATIVE makes the runtime check it. A
 *    wait that does not end within about half a second sets a status bit
 *    (kvq_stats reports KVQ_ERR_DEVICE) instead of hanging.
 *  - Multi-byte values in packed planes are little-endian.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ formats
 * A packed cache is two byte planes in row order [batch][head][position]:
 * a code plane with a fixed number of bytes per row and a scale plane with a
 * fixed number of bytes per row (kvq_row_bytes). All rounding is done in
 * float64 with one round-to-nearest-even per narrowing.
 *
 * KVQ_Q8_0    ([SV] format list). Blocks of 32: d = fp16(max|x|/127);
 *             code = x/d rounded half away from zero, clamped to +-127
 *             (zero scale -> zero codes). Row: dim int8 codes, dim/32 fp16 d.
 * KVQ_Q4_0    ([SV] format list). Blocks of 32: m = element of largest |x|
 *             (first on ties, sign kept), d = fp16(m / -8); code =
 *             clamp(floor(x/d + 1/2) + 8, 0, 15) (zero scale -> 8); value
 *             (code-8)*d. Row: dim/2 bytes (block b at bytes 16b.., byte j of a
 *             block = element 2j low nibble | element 2j+1 high nibble), then
 *             dim/32 fp16 d.
 * KVQ_LUT3    ([SV] turbo3-style LUT codebook). 128-wide rows only. 3-bit code
 *             = sign bit (top) + 2-bit magnitude index into the four fp16
 *             magnitudes of the 8-level Lloyd-Max quantizer of N(0,1)
 *             (fp16 bits 0x33D8 0x3A0C 0x3D60 0x404E). With norm = |x|_2
 *             (sequential float64 sum of squares) and t = x*sqrt(128)/norm,
 *             the index is the nearest magnitude to |t| (ties to the smaller),
 *             and the row scalar nu = fp16(norm*sqrt(128)/|LUT[codes]|_2)
 *             keeps the decoded norm. Value = nu*(+-M[idx])/sqrt(128).
 *             Row: 48 B = the 128 codes as one little-endian 384-bit string,
 *             element i at bits 3i..3i+2 (code = sign << 2 | index); scale
 *             plane: nu (fp16).
 * KVQ_LUT3_WHT ([SV] "Почему это работает для любой квантизации": turbo3
 *             rotates rows with a Walsh-Hadamard transform). LUT3 of
 *             y = H x / sqrt(128), H the 128x128 Sylvester Hadamard matrix
 *             (H[i][j] = (-1)^popcount(i & j)), computed in float64 as the
 *             butterflies (a, b) -> (a + b, a - b) for h = 1, 2, ..., 64 over
 *             pairs (j, j + h), j mod 2h < h, then one multiply by the float64
 *             nearest 1/sqrt(128); y is not rounded to float32 before LUT3.
 *             Decoding rotates the LUT3 value back with the same transform.
 *             Same row bytes as KVQ_LUT3.
 * KVQ_FP8_B128 ([MLA] BlockWise1x128). Groups of 128 along the row (the last
 *             may be shorter): s = fp32(max|x|/448); code =
 *             e4m3fn(clamp(x/s, -448, 448)) (OCP E4M3, nearest-even);
 *             zero scale -> zero codes. Row: dim e4m3 bytes, then one fp32
 *             per group.
 */
enum {
  KVQ_Q8_0 = 0,
  KVQ_Q4_0 = 1,
  KVQ_LUT3 = 2,
  KVQ_FP8_B128 = 3,
  KVQ_LUT3_WHT = 4
};

/* query element types */
enum { KVQ_Q_F32 = 0, KVQ_Q_BF16 = 1 };

/* error codes */
enum {
  KVQ_OK = 0,
  KVQ_ERR_ARG = -1,          /* null pointer, bad enum, inconsistent shapes */
  KVQ_ERR_ALIGN = -2,        /* a device pointer is not 16-byte aligned */
  KVQ_ERR_RANGE = -3,        /* ctx_len or threshold out of range; a scale overflows fp16 */
  KVQ_ERR_NONFINITE = -4,    /* NaN or infinity in packer input */
  KVQ_ERR_WORKSPACE = -5,    /* workspace missing or smaller than kvq_workspace_bytes */
  KVQ_ERR_LAUNCH = -6,       /* the HIP runtime refused a launch or copy */
  KVQ_ERR_UNSUPPORTED = -7,  /* valid request this build does not implement */
  KVQ_ERR_DEVICE = -8        /* a kernel reported a fault (see kvq_stats.status) */
};

/* Bytes per packed row of `dim` elements for `fmt`.
 * code_bytes/scale_bytes: host out-pointers. Errors: ARG (bad fmt, null),
 * UNSUPPORTED (dim not allowed for fmt: q8_0/q4_0 need dim % 32 == 0, LUT3
 * and LUT3_WHT need dim == 128, FP8 needs 1 <= dim). */
int32_t kvq_row_bytes(int32_t fmt, int32_t dim, int64_t* code_bytes, int64_t* scale_bytes);

/* Pack n_rows float32 rows of `dim` elements (host `src`, row-major) into the
 * host planes `codes` (n_rows * code_bytes) and `scales` (n_rows *
 * scale_bytes), per the format rules above. Synchronous, deterministic,
 * bit-exact with the format definition. Caller owns all buffers.
 * Errors: ARG, UNSUPPORTED, NONFINITE (any NaN/inf in src; nothing written
 * is guaranteed), RANGE (a scale overflows fp16). */
int32_t kvq_pack(int32_t fmt, const float* src, int64_t n_rows, int32_t dim,
                 uint8_t* codes, uint8_t* scales);

/* Decode packed host planes back to float32 host rows (a test and debugging
 * aid; values are the exact decoded values rounded once to float32). */
int32_t kvq_unpack(int32_t fmt, const uint8_t* codes, const uint8_t* scales,
                   int64_t n_rows, int32_t dim, float* dst);

/* The four LUT3 magnitudes as fp16 bit patterns (host out[4]). */
int32_t kvq_lut3_levels(uint16_t* out4);

/* Pack float32 rows that are in device memory straight into device planes:
 * the per-step append of a decode loop (the new token's key or value rows,
 * quantized on the GPU before the attention reads them), or a whole prefill.
 * Each row is packed exactly as kvq_pack packs it (same bytes), by a kernel
 * that shares kvq_pack's per-element and per-scale steps.
 *  src        device float32 [n_rows][dim], row-major, 4-byte aligned
 *  dst_rows   device int64 [n_rows]: the plane row each source row goes to,
 *             e.g. (b*heads + h)*capacity + position in a kvq_cache layout;
 *             NULL writes row r to plane row r (then n_rows <= cache_rows)
 *  codes, scales  device planes of cache_rows rows (kvq_row_bytes each),
 *             16-byte aligned; only the destination rows are written
 *  status     optional device int32: a row holding a NaN or infinity (1),
 *             whose scale overflows fp16 (2) or whose destination is outside
 *             [0, cache_rows) (4) is left unwritten and its bits are OR-ed in
 *  stream     hipStream_t (NULL = default stream); asynchronous
 * Errors (checked before any device work): ARG (bad fmt, null planes or
 * source, negative counts), UNSUPPORTED (dim, as kvq_row_bytes), ALIGN,
 * RANGE (dst_rows NULL and n_rows > cache_rows), LAUNCH. */
int32_t kvq_append(int32_t fmt, const float* src, int64_t n_rows, int32_t dim, const int64_t* dst_rows,
                   void* codes, void* scales, int64_t cache_rows, int32_t* status, void* stream);

/* kvq_append for a key and a value cache in one launch (a decode step's two
 * appends): k_src and v_src are both device float32 [n_rows][dim], the rows
 * go to the same dst_rows of (k_codes, k_scales) and (v_codes, v_scales),
 * each cache_rows rows of the same format and dim. Arguments, status bits
 * and errors as kvq_append. */
int32_t kvq_append_kv(int32_t fmt, const float* k_src, const float* v_src, int64_t n_rows, int32_t dim,
                      const int64_t* dst_rows, void* k_codes, void* k_scales, void* v_codes, void* v_scales,
                      int64_t cache_rows, int32_t* status, void* stream);

/* Key-block summaries for KVQ_SKIP_KEYS. For each of n_seqs consecutive
 * (sequence, head) row ranges of `capacity` rows of a packed cache and each
 * block k of 64 rows (the last one shorter when capacity % 64 != 0):
 *   out[s][k] = max over the block's rows of ||dequant(row)||,
 * each norm the square root of the float64 sum of the squared float64
 * dequantized elements added in element order (for KVQ_LUT3_WHT after the
 * inverse rotation, as kvq_unpack), the maximum rounded up to float32, so a
 * summary never understates a norm. Rows never written (zero planes) count
 * as norm 0. kvq_key_norms works on host planes (codes, scales: n_seqs *
 * capacity rows of kvq_row_bytes; out: host float[n_seqs][ceil(capacity/64)]).
 * kvq_key_norms_device computes the same bits on the GPU from device planes
 * into device `norms`, for the flat block ids in the device list `blocks`
 * (s * ceil(capacity/64) + k; n_blocks of them) or, with blocks NULL, for
 * every block: after a decode step's kvq_append_kv, pass the blocks that
 * received rows. A listed id out of range is skipped and ORs 8 into the
 * optional device int32 `status`. Asynchronous on `stream`.
 * Errors: ARG (null pointers, negative counts, capacity < 1), UNSUPPORTED
 * (fmt/dim as kvq_row_bytes), ALIGN (norms not 4-byte, blocks not 8-byte
 * aligned), LAUNCH. */
int32_t kvq_key_norms(int32_t fmt, const void* codes, const void* scales, int64_t n_seqs, int32_t capacity,
                      int32_t dim, float* out);
int32_t kvq_key_norms_device(int32_t fmt, const void* codes, const void* scales, int64_t n_seqs,
                             int32_t capacity, int32_t dim, const int64_t* blocks, int64_t n_blocks,
                             float* norms, int32_t* status, void* stream);

/* ------------------------------------------------------------------ decode */

/* A packed cache in device memory. Row r of (batch b, head h) is at
 * codes + ((b*heads + h)*capacity + r) * code_bytes, likewise for scales.
 * Both planes must be 16-byte aligned. Rows at positions >= ctx_len are never
 * read. */
typedef struct kvq_cache {
  const void* codes;
  const void* scales;
  int32_t batch;
  int32_t heads;
  int32_t dim;
  int32_t capacity;
  const float* block_norms;   /* optional device [batch][heads][ceil(capacity/64)]: the largest key
                                 norm of each block of 64 rows (kvq_key_norms, kvq_key_norms_device);
                                 read only by KVQ_SKIP_KEYS, NULL otherwise */
} kvq_cache;

typedef struct kvq_launch {
  int32_t q_heads;        /* Hq; must be a multiple of the cache's heads */
  int32_t q_dtype;        /* KVQ_Q_F32 or KVQ_Q_BF16 */
  float softmax_scale;    /* sigma; 0 selects 1/sqrt(kcache.dim) */
  int32_t v_dim;          /* latent caches (vcache == NULL): value = first v_dim dims of each key row */
  void* workspace;        /* device, >= kvq_workspace_bytes, zero-filled before its first use */
  int64_t workspace_bytes;
  void* stream;           /* hipStream_t; NULL = the default stream */
  uint32_t* mask_out;     /* optional device [batch][q_heads][ceil(ctx_len/32)]: bit i%32 of
                             word i/32 = position i kept by that head; NULL to skip */
  int32_t splits;         /* 0 = automatic; otherwise context splits per (batch, kv head) */
  int32_t flags;          /* 0 or KVQ_LAUNCH_COOPERATIVE | KVQ_SKIP_RUNNING */
  uint64_t* phase_times;  /* optional device [workgroups][16] buffer (profiling aid; NULL to skip):
                             each workgroup stores the 100 MHz device wall clock at its phase
                             boundaries (see kvq_phase_count) */
  uint8_t* key_skip_out;  /* optional device [batch][kv_heads][ceil(ctx_len/64)] (KVQ_SKIP_KEYS):
                             1 where the block's keys were left out, else 0; NULL to skip */
} kvq_launch;

/* kvq_launch.flags (bits). The workgroups of one call exchange data while they
 * run, so all of them must be resident at once; the plan never launches more
 * than one workgroup per compute unit. By default the kernel is launched
 * normally (lowest latency), and every wait is bounded (about half a second)
 * so a call that cannot get its workgroups resident, e.g. because another
 * kernel holds the compute units, ends with KVQ_ERR_DEVICE from kvq_stats
 * rather than a hang. KVQ_LAUNCH_COOPERATIVE asks the runtime to guarantee
 * co-residency (hipLaunchCooperativeKernel), at roughly 20 us extra per call.
 *
 * KVQ_SKIP_RUNNING selects the single-pass skip rule of an in-loop
 * flash-attention kernel ([SV] "Решение — не ускорять, а пропускать": the
 * skip is decided from the weights inside the loop): the context is cut into
 * the plan's splits (kvq_stats.splits; P = ceil(ctx_len / splits) rounded up
 * to a multiple of 64 positions), each walked in blocks of 64 positions, and
 * position i is kept when its weight under the softmax of its split's
 * positions up to the end of its block reaches the threshold. That weight is
 * never smaller than the normalized weight, so the kept set contains the
 * default rule's; the output still uses the normalized weights of the kept
 * positions. Grouped formats only (UNSUPPORTED for the fp8 latent).
 *
 * KVQ_TEST_WITHHOLD is a test aid for the give-up path of the bounded waits:
 * context split 0 of the first (sequence, kv head) group does not publish its
 * split statistics, and every wait gives up after about 4096 polls instead of
 * about half a second. The call still ends normally: every wait that gives up
 * sets the sticky status bit (kvq_stats then returns KVQ_ERR_DEVICE), and
 * every output element and kept mass that depended on a wait that gave up is
 * written as NaN (here: all outputs of the first group; the other groups are
 * exact). After such a call the workspace must be zero-filled again.
 *
 * KVQ_SKIP_KEYS leaves out key blocks whose weights a bound proves negligible
 * ([SV] FAQ "Почему нельзя пропускать и K-деквантизацию?": a first pass has
 * to filter key positions). It reads kcache->block_norms (required) and, for
 * each (sequence, kv head), with blocks k of 64 positions and R_k their
 * largest key norm:
 *   1. candidate blocks: R_k >= R_max / 2 (R_max over the context's blocks);
 *      they are scored first, and L_h, the log-sum-exp of head h's scores
 *      over them, is a lower bound of the head's full log-sum-exp;
 *   2. any other block is dropped, its keys never read, when for every head
 *      h of the group |B_k| * exp(sigma * ||q_h|| * R_k - L_h) <= 1e-7, |B_k|
 *      its positions inside the context (sigma * ||q_h|| * R_k bounds every
 *      score of the block, so its whole weight is at most 1e-7);
 *   3. the softmax, the keep rule and the output are then taken over the
 *      positions of the blocks not dropped; the normalized weights there are
 *      the exact ones times at most 1 / (1 - W), W <= 1e-7 per dropped block.
 * The blocks that are neither candidates nor dropped are scored after an
 * extra exchange of the candidates' statistics. Grouped formats only, not
 * with KVQ_SKIP_RUNNING (UNSUPPORTED); ARG if kcache->block_norms is NULL.
 * kvq_stats.key_rows_skipped counts the positions left out;
 * kvq_launch.key_skip_out optionally receives the dropped blocks. */
enum { KVQ_LAUNCH_COOPERATIVE = 1, KVQ_SKIP_RUNNING = 2, KVQ_TEST_WITHHOLD = 4, KVQ_SKIP_KEYS = 8 };

/* Device workspace bytes kvq_decode_attn needs for these shapes on the
 * current device (bytes: host out-pointer), for every context length from 1
 * to ctx_len: one workspace serves a decode loop whose context grows or
 * shrinks within that bound, with the same format, cache shape and launch
 * settings (splits, heads, value width). */
int32_t kvq_workspace_bytes(int32_t fmt, const kvq_cache* kcache, const kvq_launch* l,
                            int32_t ctx_len, int64_t* bytes);

/* Single-token decode attention with the sparse-V skip ([SV], section
 * "Решение — не ускорять, а пропускать"). For each sequence b and query head
 * h (kv head g = floor(h*Hkv/Hq), n = ctx_len, sigma = softmax scale):
 *   s_i = sigma * <q[b,h], dequant(K[b,g,i])>          for all i < n
 *   p_i = exp(s_i - max s) / sum_j exp(s_j - max s)    (normalized weight)
 *   out[b,h] = sum over i with p_i >= threshold of p_i * dequant(V[b,g,i])
 * No renormalization over kept positions; V rows whose weight is below the
 * threshold for every head of the group are never read. threshold = 0 gives
 * dense attention.
 *  q        device [batch][q_heads][kcache.dim], float32 or bfloat16
 *  kcache   key cache (and, when vcache is NULL, the latent the values come from)
 *  vcache   value cache with the same batch/heads/capacity, or NULL (latent)
 *  fmt      KVQ_* format of both caches
 *  ctx_len  1 <= ctx_len <= capacity
 *  threshold  0 <= threshold < 1, finite
 *  out      device float32 [batch][q_heads][value dim]
 * Asynchronous on l->stream; returns after enqueueing. Errors: ARG, ALIGN,
 * RANGE, WORKSPACE, UNSUPPORTED (shape outside the built kernels), LAUNCH.
 * Device-side faults are reported by kvq_stats.
 * Grouped formats: one launch holds at most one workgroup per compute unit
 * and keeps a split's scores (q_heads/kv_heads * positions per split floats)
 * in LDS. A call whose batch * kv_heads groups do not fit one launch under
 * both limits is enqueued as several launches on l->stream, each over an
 * equal share of the groups (in group order) with more splits per group;
 * kvq_stats.launches reports how many. UNSUPPORTED only when one group alone
 * does not fit (about 1.1 million positions at 8 query heads per kv head).
 * If a launch fails to enqueue, earlier launches of the call may have run. */
int32_t kvq_decode_attn(const void* q, const kvq_cache* kcache, const kvq_cache* vcache,
                        int32_t fmt, int32_t ctx_len, float threshold, float* out,
                        const kvq_launch* l);

/* kvq_decode_attn for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same computation, kernels and arguments, except that l->workspace and
 * l->workspace_bytes are ignored. Instead the library uses a fixed 8 MiB
 * device array of its own (one per GPU, zero when the library is loaded and
 * kept valid by the kernels from call to call; it is held until the process
 * ends). The caller still passes q, the caches and out. No call allocates.
 * Grouped-query formats only: the fp8 latent plans need far more workspace
 * (UNSUPPORTED); a plan whose workspace exceeds 8 MiB returns
 * KVQ_ERR_WORKSPACE (on a 256-CU GPU every grouped plan fits). Every call on
 * one GPU uses that GPU's array: calls that overlap on one GPU (concurrent
 * streams, or several threads) race and must be serialized by the caller.
 * kvq_stats cannot read this array's counters; a bounded wait that gives up
 * still shows as NaN in the outputs that depended on it.
 * Errors: as kvq_decode_attn, plus LAUNCH if the array's address cannot be
 * obtained. */
int32_t kvq_decode_attn_noalloc(const void* q, const kvq_cache* kcache, const kvq_cache* vcache,
                                int32_t fmt, int32_t ctx_len, float threshold, float* out,
                                const kvq_launch* l);

typedef struct kvq_stats_t {
  int64_t positions;       /* batch * kv_heads * ctx_len key rows scored */
  int64_t pairs;           /* batch * q_heads * ctx_len (head, position) weights */
  int64_t kept_pairs;      /* weights >= threshold */
  int64_t rows_fetched;    /* value rows read (kept by at least one head of the group) */
  int64_t k_bytes;         /* key bytes read (codes + scales) */
  int64_t v_bytes;         /* value bytes read */
  int64_t v_bytes_dense;   /* value bytes a dense pass reads */
  int32_t status;          /* 0 = ok; nonzero = device fault bits */
  int32_t splits;          /* context splits per (batch, kv head) used */
  int32_t batch;
  int32_t q_heads;
  int64_t live_tiles;      /* grouped formats: 64-position chunks holding a row kept by some head
                              (the chunks whose value rows are read); fp8 latent: 32-position
                              tiles re-scored because their score maximum could reach the
                              threshold (a superset of the tiles holding kept rows) */
  int32_t launches;        /* kernel launches of the call: grouped formats run in several when
                              one launch cannot hold every group (see kvq_decode_attn); the
                              fp8 latent path always uses two (scores, then output) */
  int32_t reserved;
  int64_t key_rows_skipped;  /* KVQ_SKIP_KEYS: key positions (inside the context) left out */
} kvq_stats_t;

/* Statistics of the last kvq_decode_attn on this workspace. Synchronizes
 * l->stream, then copies. kept_mass (optional host float[batch*q_heads])
 * receives sum of kept weights per head. Returns KVQ_ERR_DEVICE when the
 * call reported a fault; the workspace must then be zero-filled again. */
int32_t kvq_stats(const kvq_launch* l, kvq_stats_t* out, float* kept_mass);

/* Number of workgroups the last kvq_decode_attn on this workspace launched
 * (rows of kvq_launch.phase_times) and the number of phase stamps per row
 * (host out-pointers; synchronizes l->stream). */
int32_t kvq_phase_count(const kvq_launch* l, int32_t* workgroups, int32_t* stamps);

/* Measurement reference, not part of the attention path: read `bytes`
 * bytes (a multiple of 16) of device memory at `src` (16-byte aligned) with
 * `grid` workgroups of `threads` threads (256, 512 or 1024), workgroup g
 * taking the g-th of `grid` contiguous slices with 16-byte loads (each thread
 * issues up to eight loads before it uses the first), and XOR every 32-bit
 * word a workgroup read into sink[g] (device uint32[grid], caller-owned; zero
 * it first to read the XOR back). Timing it over the bytes of a decode call
 * gives the bandwidth a plain streaming read reaches at that size.
 * Asynchronous on `stream` (a hipStream_t, NULL: default). Errors: ARG (null
 * pointer, bytes <= 0 or not a multiple of 16, grid outside 1..2^20, another
 * workgroup size), ALIGN, LAUNCH. */
int32_t kvq_stream_read(const void* src, int64_t bytes, int32_t grid, int32_t threads, uint32_t* sink,
                        void* stream);

/* Static text for an error code. */
const char* kvq_strerror(int32_t code);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
