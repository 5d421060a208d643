// C ABI of liboscar.so: argument validation, error reporting, workspace
// sizing and kernel launches.  See include/oscar.h for the contract.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <cmath>

#include "oscar_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = 0;
  return OSCAR_OK;
}

int check_params(const oscar_params *p) {
  if (!p) return fail(OSCAR_EINVAL, "params is NULL");
  if (p->head_dim != OSCAR_HEAD_DIM) return fail(OSCAR_ENOTSUP, "head_dim must be 128 (got %d)", p->head_dim);
  if (p->num_kv_heads < 1) return fail(OSCAR_EINVAL, "num_kv_heads must be >= 1");
  if (p->num_q_heads < p->num_kv_heads || p->num_q_heads % p->num_kv_heads)
    return fail(OSCAR_EINVAL, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                p->num_q_heads, p->num_kv_heads);
  if (p->num_q_heads / p->num_kv_heads > oscar::kMaxGroupHeads)
    return fail(OSCAR_ENOTSUP, "at most %d query heads per KV head", oscar::kMaxGroupHeads);
  if (p->sink < 64 || p->sink % 64) return fail(OSCAR_ENOTSUP, "sink must be a positive multiple of 64");
  if (p->recent < 64 || p->recent % 64) return fail(OSCAR_ENOTSUP, "recent must be a positive multiple of 64");
  if (p->sink + p->recent > 4096) return fail(OSCAR_ENOTSUP, "sink + recent must be <= 4096");
  if (p->page_tokens != OSCAR_PAGE_TOKENS) return fail(OSCAR_ENOTSUP, "page_tokens must be 64");
  if (p->group != OSCAR_GROUP) return fail(OSCAR_ENOTSUP, "group must be 64");
  if (!(p->sm_scale > 0.f) || !std::isfinite(p->sm_scale)) return fail(OSCAR_EINVAL, "sm_scale must be positive and finite");
  return OSCAR_OK;
}

// Tensors whose rows the kernels read or write 16 bytes at a time.
bool misaligned(const void *ptr) { return ((uintptr_t)ptr & 15u) != 0; }

int check_pool(const oscar_params *p, const oscar_kv_pool *pool) {
  if (!pool) return fail(OSCAR_EINVAL, "pool is NULL");
  if (pool->batch < 1) return fail(OSCAR_EINVAL, "pool.batch must be >= 1");
  if (!pool->sink_k || !pool->sink_v || !pool->recent_k || !pool->recent_v || !pool->block_table ||
      !pool->sink_slot || !pool->seq_lens)
    return fail(OSCAR_EINVAL, "pool has a NULL tensor pointer");
  if (pool->max_pages < 0 || pool->n_pages < 0 || pool->n_sink_slots < 1)
    return fail(OSCAR_EINVAL, "pool sizes must be non-negative (n_sink_slots >= 1)");
  if (pool->n_pages > 0 && !pool->pages) return fail(OSCAR_EINVAL, "pool.pages is NULL");
  if (misaligned(pool->sink_k) || misaligned(pool->sink_v) || misaligned(pool->recent_k) ||
      misaligned(pool->recent_v) || misaligned(pool->pages))
    return fail(OSCAR_EINVAL, "pool tensors must be 16-byte aligned");
  (void)p;
  return OSCAR_OK;
}

int check_rot(const oscar_rotation *r) {
  if (!r || !r->U_K || !r->U_V || !r->tau_K || !r->tau_V) return fail(OSCAR_EINVAL, "rotation has a NULL pointer");
  if (misaligned(r->U_K) || misaligned(r->U_V)) return fail(OSCAR_EINVAL, "U_K/U_V must be 16-byte aligned");
  return OSCAR_OK;
}

// Decode options: NULL means every field 0 (the defaults).
int check_opts(const oscar_decode_options *o, oscar_decode_options *out) {
  *out = oscar_decode_options{0, 0, 0};
  if (!o) return OSCAR_OK;
  if (o->variant < 0 || o->variant > 1) return fail(OSCAR_EINVAL, "options.variant must be 0 (MFMA) or 1 (VALU)");
  if (o->blocks < 0 || o->blocks > 65536) return fail(OSCAR_EINVAL, "options.blocks must be in [0, 65536]");
  if (o->prefix_pages < 0) return fail(OSCAR_EINVAL, "options.prefix_pages must be >= 0");
  *out = *o;
  return OSCAR_OK;
}

// The shared-prefix options against the shape (n_pages < 0: pool not known yet).
int check_prefix(const oscar_params *p, int32_t max_pages, int32_t n_pages, const oscar_decode_options &o) {
  if (o.prefix_pages == 0) return OSCAR_OK;
  if (o.variant != 0) return fail(OSCAR_EINVAL, "options.prefix_pages needs variant 0");
  if (o.prefix_pages > max_pages) return fail(OSCAR_EINVAL, "options.prefix_pages exceeds max_pages");
  if (o.prefix_pages > oscar::kMaxPrefixPages)
    return fail(OSCAR_EINVAL, "options.prefix_pages exceeds %d", oscar::kMaxPrefixPages);
  if (n_pages == 0) return fail(OSCAR_EINVAL, "options.prefix_pages needs a pool with pages");
  return OSCAR_OK;
}

oscar::PoolView make_pv(const oscar_params *p, const oscar_kv_pool *pool) {
  oscar::PoolView v{};
  v.sink_k = pool->sink_k;
  v.sink_v = pool->sink_v;
  v.recent_k = pool->recent_k;
  v.recent_v = pool->recent_v;
  v.pages = pool->pages;
  v.block_table = pool->block_table;
  v.sink_slot = pool->sink_slot;
  v.seq_lens = pool->seq_lens;
  v.err = pool->error_flags;
  v.app_cnt = pool->append_counters;
  v.batch = pool->batch;
  v.max_pages = pool->max_pages;
  v.n_pages = pool->n_pages;
  v.n_sink_slots = pool->n_sink_slots;
  v.hkv = p->num_kv_heads;
  v.hq = p->num_q_heads;
  v.sink = p->sink;
  v.recent = p->recent;
  v.sm_scale = p->sm_scale;
  return v;
}

}  // namespace

extern "C" {

const char *oscar_last_error(void) { return g_err; }

int32_t oscar_version(void) { return 1000; }

int32_t oscar_calibrate_rotation(const oscar_params *p, const float *q_cal, int64_t n_q,
                                 const float *k_cal, const float *v_cal, int64_t n_kv,
                                 double quantile_k, double quantile_v, float *U_K, float *U_V,
                                 float *tau_K, float *tau_V) {
  int rc = check_params(p);
  if (rc) return rc;
  if (!q_cal || !k_cal || !v_cal || !U_K || !U_V || !tau_K || !tau_V)
    return fail(OSCAR_EINVAL, "calibration pointer is NULL");
  const int G = p->num_q_heads / p->num_kv_heads;
  if (n_q < 1 || n_q * G < p->head_dim) return fail(OSCAR_EINVAL, "need n_q * G >= head_dim calibration queries");
  if (n_kv < 1) return fail(OSCAR_EINVAL, "need at least one calibration key/value");
  if (!(quantile_k > 0.0 && quantile_k < 1.0) || !(quantile_v > 0.0 && quantile_v < 1.0))
    return fail(OSCAR_EINVAL, "quantiles must lie in (0, 1)");
  char msg[256] = "";
  rc = oscar::calibrate_host(p->head_dim, p->num_kv_heads, p->num_q_heads, p->sm_scale, q_cal, n_q, k_cal,
                             v_cal, n_kv, quantile_k, quantile_v, U_K, U_V, tau_K, tau_V, msg, sizeof(msg));
  if (rc) return fail(rc, "%s", msg);
  return ok();
}

int32_t oscar_calibrate_codebook(const oscar_params *p, const float *U, const float *tau, const float *x_cal,
                                 int64_t n, uint32_t *levels) {
  int rc = check_params(p);
  if (rc) return rc;
  if (!U || !tau || !x_cal || !levels) return fail(OSCAR_EINVAL, "codebook pointer is NULL");
  if (n < 1) return fail(OSCAR_EINVAL, "need at least one calibration token");
  char msg[256] = "";
  rc = oscar::calibrate_codebook_host(p->head_dim, p->num_kv_heads, U, tau, x_cal, n, levels, msg, sizeof(msg));
  if (rc) return fail(rc, "%s", msg);
  return ok();
}

int32_t oscar_quantize_append(const oscar_params *p, const oscar_rotation *rot,
                              const oscar_kv_pool *pool, const uint16_t *k_new,
                              const uint16_t *v_new, int32_t n_new, void *stream) {
  int rc = check_params(p);
  if (rc) return rc;
  if ((rc = check_rot(rot)) || (rc = check_pool(p, pool))) return rc;
  if (n_new < 1) return fail(OSCAR_EINVAL, "n_new must be >= 1");
  if (!k_new || !v_new) return fail(OSCAR_EINVAL, "k_new/v_new is NULL");
  if (misaligned(k_new) || misaligned(v_new)) return fail(OSCAR_EINVAL, "k_new/v_new must be 16-byte aligned");
  oscar::PoolView pv = make_pv(p, pool);
  oscar::RotView rv{rot->U_K, rot->U_V, rot->tau_K, rot->tau_V, rot->levels_K, rot->levels_V};
  hipError_t e = oscar::launch_append(pv, rv, k_new, v_new, n_new, (hipStream_t)stream);
  if (e != hipSuccess) return fail(OSCAR_EHIP, "append launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t oscar_decode_workspace_size(const oscar_params *p, int32_t batch, int32_t max_pages,
                                   const oscar_decode_options *opts) {
  oscar_decode_options o;
  if (check_params(p) || batch < 1 || max_pages < 0 || check_opts(opts, &o) || check_prefix(p, max_pages, -1, o))
    return 0;
  return oscar::make_decode_plan(batch, p->num_kv_heads, p->num_q_heads, max_pages, p->sink, p->recent, o.variant,
                                 o.blocks, o.prefix_pages)
      .total;
}

int32_t oscar_decode_attention(const oscar_params *p, const oscar_rotation *rot,
                               const oscar_kv_pool *pool, const uint16_t *q, float *out,
                               const oscar_decode_options *opts, void *workspace,
                               size_t workspace_bytes, void *stream) {
  int rc = check_params(p);
  if (rc) return rc;
  if ((rc = check_rot(rot)) || (rc = check_pool(p, pool))) return rc;
  oscar_decode_options o;
  if ((rc = check_opts(opts, &o)) || (rc = check_prefix(p, pool->max_pages, pool->n_pages, o))) return rc;
  if (!q || !out) return fail(OSCAR_EINVAL, "q/out is NULL");
  if (misaligned(q) || misaligned(out)) return fail(OSCAR_EINVAL, "q/out must be 16-byte aligned");
  const oscar::DecodePlan plan = oscar::make_decode_plan(pool->batch, p->num_kv_heads, p->num_q_heads,
                                                          pool->max_pages, p->sink, p->recent, o.variant, o.blocks,
                                                          o.prefix_pages);
  if (!workspace || workspace_bytes < plan.total)
    return fail(OSCAR_EWORKSPACE, "workspace of %zu bytes needed, %zu given", plan.total, workspace_bytes);
  if (((uintptr_t)workspace) & 255) return fail(OSCAR_EINVAL, "workspace must be 256-byte aligned");
  oscar::PoolView pv = make_pv(p, pool);
  oscar::RotView rv{rot->U_K, rot->U_V, rot->tau_K, rot->tau_V, rot->levels_K, rot->levels_V};
  hipError_t e = oscar::launch_decode(pv, rv, q, out, (uint8_t *)workspace,
                                      (int *)((uint8_t *)workspace + plan.off_counters), plan, o.variant,
                                      (hipStream_t)stream);
  if (e != hipSuccess) return fail(OSCAR_EHIP, "decode launch failed: %s", hipGetErrorString(e));
  return ok();
}

int32_t oscar_decode_attention_noalloc(const oscar_params *p, const oscar_rotation *rot,
                                       const oscar_kv_pool *pool, const uint16_t *q, float *out,
                                       const oscar_decode_options *opts, void *stream) {
  int rc = check_params(p);
  if (rc) return rc;
  if ((rc = check_rot(rot)) || (rc = check_pool(p, pool))) return rc;
  oscar_decode_options o;
  if ((rc = check_opts(opts, &o)) || (rc = check_prefix(p, pool->max_pages, pool->n_pages, o))) return rc;
  if (!q || !out) return fail(OSCAR_EINVAL, "q/out is NULL");
  if (misaligned(q) || misaligned(out)) return fail(OSCAR_EINVAL, "q/out must be 16-byte aligned");
  const oscar::DecodePlan plan = oscar::make_decode_plan(pool->batch, p->num_kv_heads, p->num_q_heads,
                                                          pool->max_pages, p->sink, p->recent, o.variant, o.blocks,
                                                          o.prefix_pages);
  // the plan's counters go to the buffer's counter region, everything after
  // them (from off_qconst on) to the rest of the buffer
  const size_t counters = (size_t)pool->batch * p->num_kv_heads * sizeof(int);
  const size_t cbytes = oscar::noalloc_counter_bytes();
  const size_t rest = plan.total - plan.off_qconst;
  if (counters > cbytes || rest > (size_t)OSCAR_NOALLOC_SCRATCH_BYTES - cbytes)
    return fail(OSCAR_EWORKSPACE,
                "no-alloc decode needs %zu counter bytes and %zu scratch bytes; the library holds %zu and %zu",
                counters, rest, cbytes, (size_t)OSCAR_NOALLOC_SCRATCH_BYTES - cbytes);
  uint8_t *base = nullptr;
  hipError_t e = oscar::noalloc_scratch((hipStream_t)stream, &base);
  if (e != hipSuccess) return fail(OSCAR_EHIP, "no-alloc decode buffer: %s", hipGetErrorString(e));
  oscar::PoolView pv = make_pv(p, pool);
  oscar::RotView rv{rot->U_K, rot->U_V, rot->tau_K, rot->tau_V, rot->levels_K, rot->levels_V};
  e = oscar::launch_decode(pv, rv, q, out, base + cbytes - plan.off_qconst, (int *)base, plan, o.variant,
                           (hipStream_t)stream);
  if (e != hipSuccess) return fail(OSCAR_EHIP, "decode launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t oscar_bf16_decode_workspace_size(const oscar_params *p, int32_t batch, int32_t max_pages) {
  if (check_params(p) || batch < 1 || max_pages < 0) return 0;
  return oscar::make_bf16_plan(batch, p->num_kv_heads, p->num_q_heads, max_pages).total;
}

int32_t oscar_bf16_decode_attention(const oscar_params *p, const oscar_bf16_cache *cache,
                                    const uint16_t *q, float *out, void *workspace,
                                    size_t workspace_bytes, void *stream) {
  int rc = check_params(p);
  if (rc) return rc;
  if (!cache || !cache->k_pages || !cache->v_pages || !cache->block_table || !cache->seq_lens)
    return fail(OSCAR_EINVAL, "bf16 cache has a NULL pointer");
  if (cache->batch < 1 || cache->max_pages < 0 || cache->n_pages < 0) return fail(OSCAR_EINVAL, "bad bf16 cache sizes");
  if (misaligned(cache->k_pages) || misaligned(cache->v_pages))
    return fail(OSCAR_EINVAL, "bf16 cache pages must be 16-byte aligned");
  if (!q || !out) return fail(OSCAR_EINVAL, "q/out is NULL");
  if (misaligned(q) || misaligned(out)) return fail(OSCAR_EINVAL, "q/out must be 16-byte aligned");
  const oscar::Bf16Plan plan = oscar::make_bf16_plan(cache->batch, p->num_kv_heads, p->num_q_heads, cache->max_pages);
  if (!workspace || workspace_bytes < plan.total)
    return fail(OSCAR_EWORKSPACE, "workspace of %zu bytes needed, %zu given", plan.total, workspace_bytes);
  oscar::Bf16View v{cache->k_pages, cache->v_pages, cache->block_table, cache->seq_lens, cache->error_flags,
                    cache->batch, cache->max_pages, cache->n_pages, p->num_kv_heads, p->num_q_heads, p->sm_scale};
  hipError_t e = oscar::launch_bf16_decode(v, q, out, (uint8_t *)workspace, plan, (hipStream_t)stream);
  if (e != hipSuccess) return fail(OSCAR_EHIP, "bf16 decode launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
