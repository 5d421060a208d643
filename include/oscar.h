/*
 * oscar.h -- C ABI of liboscar.so: OSCAR rotated-INT2 KV-cache decode
 * attention for AMD Instinct MI355X (gfx950).
 *
 * Sources (cited by page title and section):
 *   [A] youleyou.com article "超越 TurboQuant，显存压力终于得到缓解！Together AI
 *       最新论文 OSCAR 直接挑战 TurboQuant …", section "OSCAR 的设计思路" and the
 *       token-pool paragraphs that follow it.
 *   [B] MarkTechPost article, Chinese translation, "Together AI 开源 OSCAR：一种
 *       用于长上下文 LLM 服务的注意力感知 2 位 KV 缓存量化系统", sections
 *       "OSCAR 有何不同做法" (method), "服务系统：混合精度缓存布局" (serving),
 *       visual-guide steps 04 and 06.
 *
 * Conventions shared by every entry point
 *   - Return value: OSCAR_OK (0) or a negative OSCAR_E* code.  On error a
 *     message is available from oscar_last_error() (per thread) and nothing
 *     has been launched.  No C++ exception crosses this boundary.
 *   - Pointers inside oscar_rotation, oscar_kv_pool and oscar_bf16_cache, and
 *     the tensor arguments of the decode/append calls, are DEVICE pointers
 *     owned by the caller.  The library never allocates or frees them and
 *     keeps no reference after the call returns.  oscar_calibrate_rotation
 *     alone takes HOST pointers.
 *   - Device calls are asynchronous on `stream` (a hipStream_t; NULL = the
 *     default stream).  Faults inside a kernel surface at the caller's next
 *     synchronisation.  Conditions only the device can see (a block-table
 *     entry outside [0, n_pages), a sequence longer than the table) are
 *     skipped by the kernels and reported by OR-ing OSCAR_DEVERR_* bits into
 *     *pool->error_flags when that pointer is non-NULL.
 *   - Every float and bf16 device tensor (rotation factors, pool pages and
 *     BF16 segments, q, out, new tokens) must be 16-byte aligned, as any
 *     hipMalloc or torch allocation is; OSCAR_EINVAL otherwise.
 *   - bf16 values are passed as their uint16_t bit patterns.
 *   - All tokens are row vectors; d = head_dim = 128.
 */
#ifndef OSCAR_H
#define OSCAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  OSCAR_OK = 0,
  OSCAR_EINVAL = -1,     /* invalid argument (message says which) */
  OSCAR_ENOTSUP = -2,    /* valid but unsupported configuration */
  OSCAR_EWORKSPACE = -3, /* workspace too small */
  OSCAR_EHIP = -4        /* HIP runtime error at launch */
};

/* Bits OR-ed into *oscar_kv_pool.error_flags by the kernels. */
enum {
  OSCAR_DEVERR_PAGE = 1,     /* block-table entry outside [0, n_pages), or a shared-prefix
                                entry that differs from sequence 0's */
  OSCAR_DEVERR_LENGTH = 2,   /* sequence needs more pages than max_pages, or its history is
                                shorter than the shared prefix */
  OSCAR_DEVERR_SINKSLOT = 4  /* sink_slot entry outside [0, n_sink_slots) */
};

/* Fixed geometry of this version. */
#define OSCAR_HEAD_DIM 128
#define OSCAR_PAGE_TOKENS 64
#define OSCAR_GROUP 64
/*
 * One history page holds 64 token slots of one KV head, 4608 bytes:
 *   [   0, 2048)  K codes, token-major: row t (32 bytes) is token slot t;
 *                 byte j holds channels 4j..4j+3, channel 4j+i in bits
 *                 [2i, 2i+2).
 *   [2048, 4096)  V codes, channel-major: row c (16 bytes) is channel c;
 *                 token slot t sits in byte 4*((t>>2)&3) + (t>>4), bits
 *                 [2*(t&3), 2*(t&3)+2).  (This order lets one 32-bit load
 *                 feed a 16x16x64 int8 MFMA operand directly.)
 *   [4096, 4352)  K metadata: 64 entries of 4 bytes {s8_0, z8_0, s8_1, z8_1}
 *                 (group 0 = rotated channels 0..63, group 1 = 64..127);
 *                 token slot t is entry 4*(t&15) + (t>>4).
 *   [4352, 4608)  V metadata, same layout.
 * A page id p addresses pages + (p * num_kv_heads + h) * OSCAR_PAGE_BYTES.
 * Metadata codes are relative to the KV head's clip threshold tau (tau_K or
 * tau_V of the rotation): with a = (2 tau) / 255 and b = (2 tau) / 765 (float32
 * divisions), a group's zero is z8 * a - tau and its scale s8 * b.  Codes are
 * 0..3 and dequantise as code * scale + zero in the rotated basis.
 */
#define OSCAR_PAGE_BYTES 4608
#define OSCAR_PAGE_KCODES 0
#define OSCAR_PAGE_VCODES 2048
#define OSCAR_PAGE_KMETA 4096
#define OSCAR_PAGE_VMETA 4352

/* Shape and softmax parameters, validated on every call. */
typedef struct oscar_params {
  int32_t head_dim;     /* must be 128 */
  int32_t num_kv_heads; /* Hkv >= 1 */
  int32_t num_q_heads;  /* Hq, a multiple of Hkv; Hq/Hkv <= 16 */
  int32_t sink;         /* S0: BF16 sink tokens, multiple of 64, default 64 */
  int32_t recent;       /* W: BF16 recent-window tokens, multiple of 64, default 256;
                           sink + recent <= 4096 */
  int32_t page_tokens;  /* must be 64 */
  int32_t group;        /* quantisation group G_K, must be 64 */
  float sm_scale;       /* softmax scale, usually 1/sqrt(head_dim) */
} oscar_params;

/*
 * Per-layer rotation artifact ([B] method: R_K = U_Q H P_br, R_V = U_S H P_br;
 * [B] serving: clipping thresholds).  U_* are float32 [Hkv][d][d], row k
 * column j = component k of eigenvector j, eigenvectors ordered by
 * descending eigenvalue.  The composite rotation of a row vector x is
 * x -> bitrev(FWHT(x U) / sqrt(d)).  tau_* are float32 [Hkv], finite,
 * in (0, 60000].
 *
 * levels_K, levels_V (optional, uint32 [Hkv]; NULL = the uniform grid): the
 * 2-bit codebook of each KV head ([A] summary and outlook: a Lloyd-Max
 * codebook).  Byte k of a head's word is n_k, and code k stands for
 * zero + scale * n_k / 32 instead of zero + scale * k; the n_k are strictly
 * increasing in [0, 96].  The uniform grid is n = (0, 32, 64, 96), i.e. the
 * word 0x60402000.  A token is given the code of the level nearest to
 * u = (x - zero) / scale, the thresholds being the midpoints
 * (n_k + n_{k+1}) / 64, with a tie at the middle threshold going up and at
 * the outer ones down (on the uniform grid: u rounded half to even and
 * clamped to [0, 3]).  The same levels must be given to appends and decodes
 * of a pool.  oscar_calibrate_codebook computes them.
 */
typedef struct oscar_rotation {
  const float *U_K;
  const float *U_V;
  const float *tau_K;
  const float *tau_V;
  const uint32_t *levels_K;
  const uint32_t *levels_V;
} oscar_rotation;

#define OSCAR_UNIFORM_LEVELS 0x60402000u

/*
 * Mixed-precision KV pool of one layer ([A] token pool; [B] serving):
 * positions [0, S0) in the BF16 sink, the last W positions in the BF16
 * recent ring (slot = position mod W), everything between as rotated INT2
 * history: history index i = position - S0 lives in page
 * block_table[b][i / 64], slot i % 64.
 */
typedef struct oscar_kv_pool {
  uint16_t *sink_k;            /* bf16 [n_sink_slots][Hkv][S0][d] */
  uint16_t *sink_v;
  uint16_t *recent_k;          /* bf16 [batch][Hkv][W][d] */
  uint16_t *recent_v;
  uint8_t *pages;              /* [n_pages][Hkv][OSCAR_PAGE_BYTES] */
  const int32_t *block_table;  /* int32 [batch][max_pages] */
  const int32_t *sink_slot;    /* int32 [batch]: sink slot of each sequence */
  int32_t *seq_lens;           /* int32 [batch]: tokens currently stored */
  int32_t *error_flags;        /* optional int32[1], OSCAR_DEVERR_* bits */
  int32_t *append_counters;    /* optional int32 [batch], zero-filled by the caller
                                  once; single-token appends use it to let the
                                  last block of a sequence advance seq_lens, and
                                  leave it zero.  NULL selects a two-launch path. */
  int32_t batch;
  int32_t max_pages;
  int32_t n_pages;
  int32_t n_sink_slots;
} oscar_kv_pool;

/*
 * Offline calibration of one layer ([B] method; [B] guide step 04).  HOST
 * pointers, synchronous, float64 internally.
 *   q_cal [Hq][n_q][d], k_cal and v_cal [Hkv][n_kv][d] (float32 holding bf16
 *   values).  For each KV head: C_Q = uncentred covariance of the n_q * G
 *   query rows of its G query heads; C_S = (1/(n_q G)) sum_h (S_h V)^T (S_h V)
 *   with S_h = softmax(sm_scale Q_h K^T) over the calibration keys;
 *   U = eigenvectors by descending eigenvalue, each column's largest-|.|
 *   entry positive; tau = quantile (linear interpolation) of |x R| over all
 *   rotated calibration entries, R built from the float32 U.
 * Outputs U_K, U_V [Hkv][d][d] and tau_K, tau_V [Hkv].  OSCAR_EINVAL if
 * n_q * G < d, n_kv < 1, a quantile is outside (0, 1), or a spectrum has a
 * relative eigen-gap below 1e-10 (basis not unique).
 */
int32_t oscar_calibrate_rotation(const oscar_params *p, const float *q_cal, int64_t n_q,
                                 const float *k_cal, const float *v_cal, int64_t n_kv,
                                 double quantile_k, double quantile_v, float *U_K, float *U_V,
                                 float *tau_K, float *tau_V);

/*
 * Offline Lloyd-Max codebook of one tensor (keys or values) of one layer
 * ([A] summary and outlook).  HOST pointers, synchronous, float64 Lloyd-Max
 * iteration.  U [Hkv][d][d] and tau [Hkv] are that tensor's rotation factor
 * and clip threshold (as in oscar_rotation); x_cal [Hkv][n][d] are float32
 * holding the bf16 calibration tokens.  Every calibration token goes through
 * the write path up to its codes (rotation, clip, 8-bit zero and scale per
 * 64-channel group, exactly as an append computes them); the normalised
 * values u = (x - zero) / scale of the groups whose scale is not zero feed
 * a 4-level Lloyd-Max quantiser started from (0, 1, 2, 3) (nearest-level
 * cells, cell means, until no level moves by more than 1e-12; an empty cell
 * keeps its level).  Each level is rounded to the nearest 1/32 (half to
 * even), clamped to [0, 96] and the four made strictly increasing (each
 * raised to one step above the one below, then lowered to leave one step
 * for each above).  Output: levels [Hkv] in the format of
 * oscar_rotation.levels_K.  OSCAR_EINVAL for NULL pointers or n < 1.
 */
int32_t oscar_calibrate_codebook(const oscar_params *p, const float *U, const float *tau, const float *x_cal,
                                 int64_t n, uint32_t *levels);

/*
 * Append n_new tokens to every sequence of the pool ([A] token pool: new
 * tokens enter the recent window and the oldest recent token is rotated,
 * clipped, quantised, packed and demoted by a fused write kernel).
 *   k_new, v_new: bf16 [batch][n_new][Hkv][d].
 * Sequence b receives positions seq_lens[b] .. seq_lens[b]+n_new-1 (read on
 * the device).  Every position that leaves the recent window -- old ring
 * tokens and new tokens alike -- is written to history exactly as n_new
 * single-token appends would write it (bit for bit), then seq_lens[b] grows
 * by n_new.  The pages the new history needs must already be in the block
 * table.  Concurrent appends that share a target page race.
 */
int32_t oscar_quantize_append(const oscar_params *p, const oscar_rotation *rot,
                              const oscar_kv_pool *pool, const uint16_t *k_new,
                              const uint16_t *v_new, int32_t n_new, void *stream);

/*
 * Per-call choices of the decode kernels.  Pass NULL for the defaults
 * (every field 0).  Nothing is kept between calls: the library holds no
 * process-wide decode settings.
 *   variant: 0 = MFMA int8 history scan (default), one workgroup per
 *            (sequence, KV head, split);
 *            1 = VALU history scan (float arithmetic, reference speed), on
 *            the same grid after a query-preparation kernel.
 *            OSCAR_EINVAL for other values.
 *   blocks:  history-scan workgroups the split grid aims for: each
 *            (sequence, KV head) gets ceil(blocks / (batch * Hkv)) splits,
 *            capped so every wave keeps at least one page.  0 aims for one
 *            workgroup per compute unit (256).  Results differ only in
 *            floating-point summation order.  OSCAR_EINVAL outside
 *            [0, 65536].
 *   prefix_pages: shared-prefix decode ([A] serving with a prefix cache:
 *            many sequences on the same prompt pages).  0 (default): every
 *            sequence scans all of its history pages.  P > 0: the first P
 *            history pages of every sequence in the batch are the same
 *            physical pages (equal block-table entries) and every sequence
 *            holds at least 64 P history tokens.  Those P pages are then
 *            read once per KV head for up to 8 sequences at a time: one
 *            workgroup streams each page into LDS and each of its waves
 *            scores it for one sequence's query heads; the workgroups of
 *            the other sequences of the same pages run on the same XCD, so
 *            HBM serves each page once.  Each sequence's own scan covers
 *            pages P.. only, and one merge combines both.  Needs variant 0,
 *            P <= max_pages, P <= 131072 and a pool with pages;
 *            OSCAR_EINVAL otherwise.
 *            On the device, a sequence shorter than the prefix sets
 *            OSCAR_DEVERR_LENGTH and one whose entries differ from sequence
 *            0's sets OSCAR_DEVERR_PAGE (the pages of sequence 0 are used).
 * The workspace size depends on all three, so size it with the same options.
 */
typedef struct oscar_decode_options {
  int32_t variant;
  int32_t blocks;
  int32_t prefix_pages;
} oscar_decode_options;

/*
 * Decode attention of one query token per sequence over the whole pool
 * ([A] token pool: INT2 and BF16 segments, merged by online softmax; [B]
 * serving: read path).  q: bf16 [batch][Hq][d]; out: float32 [batch][Hq][d]
 * = softmax(sm_scale q K^T) V over every stored token, with history keys
 * and values dequantised and inverse-rotated (computed as (q R_K) against
 * the rotated codes and R_V^T applied once to the merged history output).
 * Query head h reads KV head h / (Hq/Hkv).  seq_lens is read on the device;
 * a sequence of length 0 yields zeros.  opts: NULL or the kernel choices
 * above.  workspace: device memory of at least
 * oscar_decode_workspace_size(p, batch, max_pages, opts) bytes, 256-byte
 * aligned, ZERO-FILLED by the caller before its first use.  It holds
 * completion counters that every call returns to zero, so it can be reused
 * without clearing; calls that share a workspace must not overlap (same
 * stream, or ordered).  With variant 0 the call is one kernel launch on
 * `stream`.
 */
int32_t oscar_decode_attention(const oscar_params *p, const oscar_rotation *rot,
                               const oscar_kv_pool *pool, const uint16_t *q, float *out,
                               const oscar_decode_options *opts, void *workspace,
                               size_t workspace_bytes, void *stream);

/* Workspace bytes oscar_decode_attention needs for this shape and these
 * options (NULL = defaults); 0 for invalid parameters or options. */
size_t oscar_decode_workspace_size(const oscar_params *p, int32_t batch, int32_t max_pages,
                                   const oscar_decode_options *opts);

/*
 * oscar_decode_attention without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same arguments, results and
 * errors as oscar_decode_attention with the same options; it calls no
 * allocating routine.  Instead of a workspace it uses a buffer the library
 * holds in each GPU's memory for the life of the process,
 * OSCAR_NOALLOC_SCRATCH_BYTES bytes: the first 64 KiB hold completion
 * counters (at most 16384 sequence x KV-head pairs), the rest one call's
 * query operands and partials, i.e. oscar_decode_workspace_size(...) minus
 * the counters.  Larger shapes are rejected with OSCAR_EWORKSPACE before
 * anything is launched.  Every call on one GPU shares that GPU's buffer, so
 * calls that overlap on one GPU (different streams or threads without
 * ordering) race; calls ordered on one stream do not.  The first call on a
 * device enqueues a clear of the counters on `stream` before its decode.
 */
#define OSCAR_NOALLOC_SCRATCH_BYTES (32u << 20)
int32_t oscar_decode_attention_noalloc(const oscar_params *p, const oscar_rotation *rot,
                                       const oscar_kv_pool *pool, const uint16_t *q, float *out,
                                       const oscar_decode_options *opts, void *stream);

/*
 * In-house BF16 decode baseline on a paged all-BF16 cache (the comparison
 * every speedup is quoted against): k_pages, v_pages bf16
 * [n_pages][Hkv][64][d]; token position t of sequence b lives in page
 * block_table[b][t / 64], slot t % 64.  Same q/out and workspace
 * conventions as oscar_decode_attention (zero-filled before first use).
 */
typedef struct oscar_bf16_cache {
  const uint16_t *k_pages;
  const uint16_t *v_pages;
  const int32_t *block_table; /* int32 [batch][max_pages] */
  const int32_t *seq_lens;    /* int32 [batch] */
  int32_t *error_flags;       /* optional */
  int32_t batch;
  int32_t max_pages;
  int32_t n_pages;
} oscar_bf16_cache;

int32_t oscar_bf16_decode_attention(const oscar_params *p, const oscar_bf16_cache *cache,
                                    const uint16_t *q, float *out, void *workspace,
                                    size_t workspace_bytes, void *stream);

size_t oscar_bf16_decode_workspace_size(const oscar_params *p, int32_t batch, int32_t max_pages);

/* Message of the last error on the calling thread ("" if none). */
const char *oscar_last_error(void);

/* Library version, e.g. 1000 for 0.1.0. */
int32_t oscar_version(void);

#ifdef __cplusplus
}
#endif

#endif /* OSCAR_H */
