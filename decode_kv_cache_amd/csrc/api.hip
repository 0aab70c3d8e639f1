// Host side of the C ABI declared in include/kara.h: argument checks,
// geometry, and the launches of the gfx950 kernels.
#include <math.h>
#include <rocprofiler-sdk-roctx/roctx.h>

#include "kara_device.h"

namespace kara {
hipError_t launch_score(const Geo& g, int dtype, const void* q, const void* kc, const int32_t* tables,
                        const int32_t* prior, float* scores, float* ws, hipStream_t st);
size_t score_workspace_bytes(const Geo& g, int dtype);
bool fused_score_supported(const Geo& g, int dtype);
hipError_t launch_select(const Geo& g, int gap, const float* scores, int32_t* kept, uint8_t* mask, hipStream_t st);
hipError_t launch_compact(const Geo& g, int dtype, void* kc, void* vc, int32_t* tables, const int32_t* prior,
                          int32_t* seq_lens, const int32_t* kept, int32_t* freed, int32_t* num_freed,
                          int max_freed, const int32_t* tails, hipStream_t st);
hipError_t launch_validate(const Geo& g, const int32_t* tables, const int32_t* prior, int32_t* bad,
                           hipStream_t st);
size_t decode_attn_workspace_bytes(const Geo& g);
hipError_t launch_pipeline(const Geo& g, const void* q, void* kc, void* vc, int32_t* tables, const int32_t* prior,
                           float* scores, int32_t* kept, uint8_t* mask, int32_t* seq_lens, int32_t* freed,
                           int32_t* num_freed, int max_freed, int32_t* done, hipStream_t st);
int decode_attn_splits(const Geo& g);
bool small_score_supported(const Geo& g, int dtype);
bool pipeline_supported(const Geo& g, int dtype);
hipError_t launch_pipeline_any(const Geo& g, int dtype, const void* q, void* kc, void* vc, int32_t* tables,
                               const int32_t* prior, float* scores, int32_t* kept, uint8_t* mask, int32_t* seq_lens,
                               int32_t* freed, int32_t* num_freed, int max_freed, int32_t* done, hipStream_t st);
hipError_t launch_pipeline_noalloc(const Geo& g, int dtype, const void* q, void* kc, void* vc, int32_t* tables,
                                   const int32_t* prior, float* scores, int32_t* kept, uint8_t* mask,
                                   int32_t* seq_lens, int32_t* freed, int32_t* num_freed, int max_freed,
                                   hipStream_t st);
hipError_t launch_decode_attn(const Geo& g, int dtype, const void* q, const void* kc, const void* vc,
                              const int32_t* tables, const int32_t* lens, float* out, float* ws, hipStream_t st);
}  // namespace kara

namespace {

thread_local int g_last_hip = 0;

bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int check(const kara_config* c) {
  if (!c) return KARA_ENULL;
  if (c->num_seqs < 0 || c->num_layers < 1 || c->num_q_heads < 1 || c->num_kv_heads < 1) return KARA_EINVAL;
  if (c->num_q_heads % c->num_kv_heads) return KARA_EINVAL;
  if (c->head_dim != 64 && c->head_dim != 128) return KARA_EINVAL;
  if (c->window < 1 || c->window > 8192) return KARA_EINVAL;
  // query rows per unit (G * W) are counted in int32 by the kernels
  if ((long long)(c->num_q_heads / c->num_kv_heads) * c->window > (1LL << 24)) return KARA_EINVAL;
  if (c->budget < 1 || c->budget > c->window) return KARA_EINVAL;
  if (c->seeds < 0 || c->radius < 0 || c->radius > c->window) return KARA_EINVAL;
  if ((long long)c->seeds * (2LL * c->radius + 1) > c->budget) return KARA_EINVAL;
  if (!pow2(c->block_size) || c->block_size > 256) return KARA_EINVAL;
  if (c->dtype != KARA_BF16 && c->dtype != KARA_F32) return KARA_EINVAL;
  if (c->max_blocks_per_seq < 1 || c->num_blocks < 0) return KARA_EINVAL;
  if (c->num_seqs > 0 && c->num_blocks < 1) return KARA_EINVAL;   // a window needs at least one block
  if (c->num_blocks > 0x7fffffffLL) return KARA_EINVAL;            // block ids are int32
  if ((long long)c->window > (long long)c->max_blocks_per_seq * c->block_size) return KARA_EINVAL;
  // logical positions, and positions plus a step or a split, stay inside int32
  if ((long long)c->max_blocks_per_seq * c->block_size > (1LL << 30)) return KARA_EINVAL;
  const long long units = (long long)c->num_seqs * c->num_layers * c->num_kv_heads;
  if (units > 0x3fffffffLL) return KARA_EINVAL;
  return KARA_OK;
}

kara::Geo geo(const kara_config* c) {
  kara::Geo g;
  g.S = c->num_seqs;
  g.Lyr = c->num_layers;
  g.Hq = c->num_q_heads;
  g.Hkv = c->num_kv_heads;
  g.G = c->num_q_heads / c->num_kv_heads;
  g.D = c->head_dim;
  g.W = c->window;
  g.B = c->budget;
  g.seeds = c->seeds;
  g.radius = c->radius;
  g.bs = c->block_size;
  g.bs_shift = __builtin_ctz((unsigned)c->block_size);
  g.max_blocks = c->max_blocks_per_seq;
  g.nblocks = c->num_blocks;
  g.GW = g.G * g.W;
  g.GWp = (g.GW + 31) & ~31;
  g.alpha = (float)(1.4426950408889634 / sqrt((double)g.D));
  return g;
}

// A roctx range around one entry point's enqueue work, named after the entry
// point, so host-side traces (rocprofv3 --marker-trace) show each call.
struct Range {
  explicit Range(const char* name) { roctxRangePushA(name); }
  ~Range() { roctxRangePop(); }
  Range(const Range&) = delete;
  Range& operator=(const Range&) = delete;
};

int hip_status(hipError_t e) {
  if (e == hipSuccess) return KARA_OK;
  g_last_hip = (int)e;
  return KARA_EHIP;
}

}  // namespace

extern "C" {

int kara_check_config(const kara_config* cfg) {
  const int s = check(cfg);
  return s == KARA_ENULL ? KARA_EINVAL : s;
}

size_t kara_workspace_bytes(const kara_config* cfg) {
  if (check(cfg) != KARA_OK) return 0;
  return kara::score_workspace_bytes(geo(cfg), cfg->dtype);
}

int kara_score_passes(const kara_config* cfg) {
  if (check(cfg) != KARA_OK) return 0;
  const kara::Geo g = geo(cfg);
  return kara::fused_score_supported(g, cfg->dtype) || kara::small_score_supported(g, cfg->dtype) ? 1 : 2;
}

int32_t kara_max_freed(const kara_config* cfg) {
  if (check(cfg) != KARA_OK) return 0;
  return (cfg->window + cfg->block_size - 1) / cfg->block_size + 1;
}

int kara_score_window(const kara_config* cfg, const void* q, const void* k_cache, const int32_t* block_tables,
                      const int32_t* prior_lens, float* scores, void* workspace, size_t workspace_bytes,
                      void* stream) {
  const Range range("kara_score_window");
  int s = check(cfg);
  if (s) return s;
  if (cfg->num_seqs == 0) return KARA_OK;
  if (!q || !k_cache || !block_tables || !prior_lens || !scores) return KARA_ENULL;
  const kara::Geo g = geo(cfg);
  const size_t need = kara::score_workspace_bytes(g, cfg->dtype);
  if (need && (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255))) return KARA_EWORKSPACE;
  return hip_status(kara::launch_score(g, cfg->dtype, q, k_cache, block_tables, prior_lens, scores,
                                       (float*)workspace, (hipStream_t)stream));
}

int kara_select_chunks(const kara_config* cfg, const float* scores, int32_t* kept, uint8_t* mask, void* stream) {
  const Range range("kara_select_chunks");
  int s = check(cfg);
  if (s) return s;
  if (cfg->num_seqs == 0) return KARA_OK;
  if (!scores || !kept) return KARA_ENULL;
  return hip_status(kara::launch_select(geo(cfg), 0, scores, kept, mask, (hipStream_t)stream));
}

int64_t kara_chunk_bound(const kara_config* cfg, int32_t gap) {
  if (!cfg || cfg->seeds < 0 || cfg->radius < 0 || gap < 0) return -1;
  const int64_t s = cfg->seeds, r = cfg->radius, extra = (int64_t)gap - 2 * r;
  return s * (2 * r + 1) + (s > 1 ? s - 1 : 0) * (extra > 0 ? extra : 0);
}

int kara_select_chunks_bridged(const kara_config* cfg, int32_t gap, const float* scores, int32_t* kept,
                               uint8_t* mask, void* stream) {
  const Range range("kara_select_chunks_bridged");
  int s = check(cfg);
  if (s) return s;
  if (gap < 0 || gap > cfg->window || kara_chunk_bound(cfg, gap) > cfg->budget) return KARA_EINVAL;
  if (cfg->num_seqs == 0) return KARA_OK;
  if (!scores || !kept) return KARA_ENULL;
  return hip_status(kara::launch_select(geo(cfg), gap, scores, kept, mask, (hipStream_t)stream));
}

int kara_compress_fused_supported(const kara_config* cfg) {
  if (check(cfg) != KARA_OK) return 0;
  return kara::pipeline_supported(geo(cfg), cfg->dtype) ? 1 : 0;
}

int kara_compress_fused(const kara_config* cfg, const void* q, void* k_cache, void* v_cache, int32_t* block_tables,
                        const int32_t* prior_lens, float* scores, int32_t* kept, uint8_t* mask, int32_t* seq_lens,
                        int32_t* freed_blocks, int32_t* num_freed, int32_t* done, void* stream) {
  const Range range("kara_compress_fused");
  int s = check(cfg);
  if (s) return s;
  const kara::Geo g = geo(cfg);
  if (!kara::pipeline_supported(g, cfg->dtype)) return KARA_ENOTIMPL;
  if (cfg->num_seqs == 0) return KARA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !prior_lens || !scores || !kept || !seq_lens || !freed_blocks ||
      !num_freed || !done)
    return KARA_ENULL;
  return hip_status(kara::launch_pipeline_any(g, cfg->dtype, q, k_cache, v_cache, block_tables, prior_lens, scores,
                                              kept, mask, seq_lens, freed_blocks, num_freed, kara_max_freed(cfg),
                                              done, (hipStream_t)stream));
}

int kara_compress_fused_noalloc(const kara_config* cfg, const void* q, void* k_cache, void* v_cache,
                                int32_t* block_tables, const int32_t* prior_lens, float* scores, int32_t* kept,
                                uint8_t* mask, int32_t* seq_lens, int32_t* freed_blocks, int32_t* num_freed,
                                void* stream) {
  const Range range("kara_compress_fused_noalloc");
  int s = check(cfg);
  if (s) return s;
  const kara::Geo g = geo(cfg);
  if (!kara::pipeline_supported(g, cfg->dtype)) return KARA_ENOTIMPL;
  if (cfg->num_seqs == 0) return KARA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !prior_lens || !scores || !kept || !seq_lens || !freed_blocks ||
      !num_freed)
    return KARA_ENULL;
  if (cfg->num_seqs > KARA_NOALLOC_MAX_SEQS) return KARA_ESCRATCH;
  if (stream) {   // the scratch address is per device: the stream must run on the current one
    int cur = -1, sdev = -1;
    if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess)
      return KARA_EINVAL;
    if (cur != sdev) return KARA_EINVAL;
  }
  return hip_status(kara::launch_pipeline_noalloc(g, cfg->dtype, q, k_cache, v_cache, block_tables, prior_lens, scores, kept,
                                                  mask, seq_lens, freed_blocks, num_freed, kara_max_freed(cfg),
                                                  (hipStream_t)stream));
}

size_t kara_decode_attention_workspace_bytes(const kara_config* cfg) {
  if (check(cfg) != KARA_OK) return 0;
  return kara::decode_attn_workspace_bytes(geo(cfg));
}

int kara_decode_attention_splits(const kara_config* cfg) {
  if (check(cfg) != KARA_OK) return 0;
  return kara::decode_attn_splits(geo(cfg));
}

int kara_decode_attention(const kara_config* cfg, const void* q_dec, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* seq_lens, float* out, void* workspace,
                          size_t workspace_bytes, void* stream) {
  const Range range("kara_decode_attention");
  int s = check(cfg);
  if (s) return s;
  if (cfg->num_seqs == 0) return KARA_OK;
  if (!q_dec || !k_cache || !v_cache || !block_tables || !seq_lens || !out) return KARA_ENULL;
  const kara::Geo g = geo(cfg);
  const size_t need = kara::decode_attn_workspace_bytes(g);
  if (need && (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255))) return KARA_EWORKSPACE;
  return hip_status(kara::launch_decode_attn(g, cfg->dtype, q_dec, k_cache, v_cache, block_tables, seq_lens, out,
                                             (float*)workspace, (hipStream_t)stream));
}

int kara_compact_paged(const kara_config* cfg, void* k_cache, void* v_cache, int32_t* block_tables,
                       const int32_t* prior_lens, int32_t* seq_lens, const int32_t* kept, int32_t* freed_blocks,
                       int32_t* num_freed, void* stream) {
  const Range range("kara_compact_paged");
  int s = check(cfg);
  if (s) return s;
  if (cfg->num_seqs == 0) return KARA_OK;
  if (!k_cache || !v_cache || !block_tables || !prior_lens || !seq_lens || !kept || !freed_blocks || !num_freed)
    return KARA_ENULL;
  return hip_status(kara::launch_compact(geo(cfg), cfg->dtype, k_cache, v_cache, block_tables, prior_lens,
                                         seq_lens, kept, freed_blocks, num_freed, kara_max_freed(cfg), nullptr,
                                         (hipStream_t)stream));
}

int kara_compact_paged_tail(const kara_config* cfg, void* k_cache, void* v_cache, int32_t* block_tables,
                            const int32_t* prior_lens, const int32_t* tail_lens, int32_t* seq_lens,
                            const int32_t* kept, int32_t* freed_blocks, int32_t* num_freed, void* stream) {
  const Range range("kara_compact_paged_tail");
  int s = check(cfg);
  if (s) return s;
  if (cfg->num_seqs == 0) return KARA_OK;
  if (!k_cache || !v_cache || !block_tables || !prior_lens || !tail_lens || !seq_lens || !kept || !freed_blocks ||
      !num_freed)
    return KARA_ENULL;
  return hip_status(kara::launch_compact(geo(cfg), cfg->dtype, k_cache, v_cache, block_tables, prior_lens,
                                         seq_lens, kept, freed_blocks, num_freed, kara_max_freed(cfg), tail_lens,
                                         (hipStream_t)stream));
}

int kara_validate_tables(const kara_config* cfg, const int32_t* block_tables, const int32_t* prior_lens,
                         int32_t* bad_seqs, void* stream) {
  const Range range("kara_validate_tables");
  int s = check(cfg);
  if (s) return s;
  if (!bad_seqs || (cfg->num_seqs > 0 && (!block_tables || !prior_lens))) return KARA_ENULL;
  return hip_status(kara::launch_validate(geo(cfg), block_tables, prior_lens, bad_seqs, (hipStream_t)stream));
}

const char* kara_status_str(int status) {
  switch (status) {
    case KARA_OK: return "ok";
    case KARA_EINVAL: return "invalid configuration or argument";
    case KARA_ENULL: return "required pointer is NULL";
    case KARA_EWORKSPACE: return "workspace missing, misaligned or too small";
    case KARA_EHIP: return "HIP runtime error while enqueueing";
    case KARA_ENOTIMPL: return "valid request this library does not support";
    case KARA_ESCRATCH: return "more sequences than the fixed scratch of an allocation-free entry point holds";
    default: return "unknown status";
  }
}

int kara_last_hip_error(void) { return g_last_hip; }

}  // extern "C"
