// Drives every entry point of the C ABI through its host-side checks: invalid
// and extreme configurations, NULL and fake pointers on the rejection paths,
// valid calls over many geometries that reach the (stand-in) launchers, and
// launches the stand-in runtime refuses (KARA_EHIP).
// Exit status 0 when every returned status is the documented one.
#include <limits.h>
#include <stdio.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "kara.h"

extern int g_launches;
extern int g_fail_launch;
static int fails = 0;

#define EXPECT(expr, want)                                                          \
  do {                                                                              \
    const long long got_ = (long long)(expr);                                       \
    if (got_ != (long long)(want)) {                                                \
      fprintf(stderr, "line %d: %s = %lld, want %lld\n", __LINE__, #expr, got_,     \
              (long long)(want));                                                   \
      ++fails;                                                                      \
    }                                                                               \
  } while (0)

static kara_config base() {
  kara_config c = {64, 32, 32, 8, 128, 1024, 204, 8, 5, 16, KARA_BF16, 4096, 100000};
  return c;
}

int main() {
  void* p = (void*)0x1000;   // never dereferenced: every call below stops on the host or at a stand-in launcher
  int32_t* ip = (int32_t*)0x1000;
  float* fp = (float*)0x1000;
  uint8_t* bp = (uint8_t*)0x1000;
  const int32_t extremes[] = {INT_MIN, -1, 0, 1, 2, 3, 7, 16, 17, 63, 64, 65, 127, 128, 129, 255, 256, 257,
                              1023, 1024, 1025, 8191, 8192, 8193, 65536, 1 << 30, INT_MAX};
  const int nx = sizeof(extremes) / sizeof(extremes[0]);
  // every int32 field through the extremes: check_config and every entry point agree
  for (int f = 0; f < 12; ++f) {
    for (int i = 0; i < nx; ++i) {
      kara_config c = base();
      int32_t* fields = &c.num_seqs;
      fields[f] = extremes[i];
      const int st = kara_check_config(&c);
      if (st != KARA_OK && st != KARA_EINVAL) ++fails;
      const int want = st == KARA_OK ? KARA_ENULL : KARA_EINVAL;
      if (c.num_seqs != 0 || st != KARA_OK) {
        EXPECT(kara_score_window(&c, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL), want);
        EXPECT(kara_select_chunks(&c, NULL, NULL, NULL, NULL), want);
        EXPECT(kara_compact_paged(&c, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL), want);
        EXPECT(kara_decode_attention(&c, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL), want);
      }
      kara_workspace_bytes(&c);
      kara_max_freed(&c);
      kara_score_passes(&c);
      kara_compress_fused_supported(&c);
      kara_decode_attention_workspace_bytes(&c);
      kara_decode_attention_splits(&c);
      for (int j = 0; j < nx; ++j) kara_chunk_bound(&c, extremes[j]);
    }
  }
  // num_blocks (int64) extremes
  const int64_t nbs[] = {LLONG_MIN, -1, 0, 1, 0x7fffffffLL, 0x80000000LL, LLONG_MAX};
  for (int i = 0; i < 7; ++i) {
    kara_config c = base();
    c.num_blocks = nbs[i];
    const int st = kara_check_config(&c);
    EXPECT(st, (nbs[i] >= 1 && nbs[i] <= 0x7fffffffLL) ? KARA_OK : KARA_EINVAL);
  }
  // NULL configuration
  EXPECT(kara_check_config(NULL), KARA_EINVAL);
  EXPECT(kara_score_window(NULL, p, p, ip, ip, fp, p, 0, NULL), KARA_ENULL);
  EXPECT(kara_compress_fused_noalloc(NULL, p, p, p, ip, ip, fp, ip, bp, ip, ip, ip, NULL), KARA_ENULL);
  EXPECT(kara_chunk_bound(NULL, 0), -1);
  // workspace checks
  {
    kara_config c = base();
    c.window = 2048;
    c.budget = 410;
    const size_t need = kara_workspace_bytes(&c);
    EXPECT(need > 0, 1);
    EXPECT(kara_score_window(&c, p, p, ip, ip, fp, NULL, need, NULL), KARA_EWORKSPACE);
    EXPECT(kara_score_window(&c, p, p, ip, ip, fp, p, need - 1, NULL), KARA_EWORKSPACE);
    EXPECT(kara_score_window(&c, p, p, ip, ip, fp, (char*)p + 16, need, NULL), KARA_EWORKSPACE);
    EXPECT(kara_score_window(&c, p, p, ip, ip, fp, p, need, NULL), KARA_OK);
  }
  // allocation-free pipeline: the fixed scratch limit
  {
    kara_config c = base();
    c.num_layers = 1;
    c.num_seqs = KARA_NOALLOC_MAX_SEQS;
    EXPECT(kara_compress_fused_noalloc(&c, p, p, p, ip, ip, fp, ip, bp, ip, ip, ip, NULL), KARA_OK);
    c.num_seqs = KARA_NOALLOC_MAX_SEQS + 1;
    EXPECT(kara_compress_fused_noalloc(&c, p, p, p, ip, ip, fp, ip, bp, ip, ip, ip, NULL), KARA_ESCRATCH);
    c.window = 2048;
    c.num_seqs = 1;
    EXPECT(kara_compress_fused_noalloc(&c, p, p, p, ip, ip, fp, ip, bp, ip, ip, ip, NULL), KARA_ENOTIMPL);
  }
  // valid calls over many geometries reach the launchers
  const int windows[] = {1, 2, 17, 128, 1024, 1025, 2048, 4096, 8192};
  const int bss[] = {1, 2, 16, 64, 256};
  const int hds[] = {64, 128};
  int calls = 0;
  for (int wi = 0; wi < 9; ++wi)
    for (int bi = 0; bi < 5; ++bi)
      for (int hi = 0; hi < 2; ++hi)
        for (int dt = 0; dt < 2; ++dt) {
          kara_config c = base();
          c.num_seqs = 3;
          c.num_layers = 2;
          c.num_q_heads = 12;
          c.num_kv_heads = 4;
          c.window = windows[wi];
          c.budget = windows[wi] > 1 ? windows[wi] / 2 : 1;
          c.seeds = 1;
          c.radius = 0;
          c.block_size = bss[bi];
          c.head_dim = hds[hi];
          c.dtype = dt;
          c.max_blocks_per_seq = (windows[wi] + 3 * bss[bi] - 1) / bss[bi] + 2;
          c.num_blocks = 3 * c.max_blocks_per_seq;
          EXPECT(kara_check_config(&c), KARA_OK);
          const size_t ws = kara_workspace_bytes(&c);
          EXPECT(kara_score_window(&c, p, p, ip, ip, fp, ws ? p : NULL, ws, NULL), KARA_OK);
          EXPECT(kara_select_chunks(&c, fp, ip, bp, NULL), KARA_OK);
          EXPECT(kara_select_chunks_bridged(&c, 0, fp, ip, NULL, NULL), KARA_OK);
          EXPECT(kara_compact_paged(&c, p, p, ip, ip, ip, ip, ip, ip, NULL), KARA_OK);
          EXPECT(kara_compact_paged_tail(&c, p, p, ip, ip, ip, ip, ip, ip, ip, NULL), KARA_OK);
          EXPECT(kara_compact_paged_tail(&c, p, p, ip, ip, NULL, ip, ip, ip, ip, NULL), KARA_ENULL);
          EXPECT(kara_validate_tables(&c, ip, ip, ip, NULL), KARA_OK);
          EXPECT(kara_decode_attention(&c, p, p, p, ip, ip, fp, NULL, 0, NULL), KARA_OK);
          const int fused = kara_compress_fused_supported(&c);
          EXPECT(kara_compress_fused(&c, p, p, p, ip, ip, fp, ip, bp, ip, ip, ip, ip, NULL),
                 fused ? KARA_OK : KARA_ENOTIMPL);
          calls += 7 + fused;
        }
  EXPECT(g_launches, calls + 1 + 1);   // + the workspace and scratch-limit calls that reached a launcher
  // a launch the runtime refuses comes back as KARA_EHIP with the HIP code kept for kara_last_hip_error
  {
    kara_config c = base();
    g_fail_launch = 1;
    EXPECT(kara_last_hip_error(), 0);
    EXPECT(kara_score_window(&c, p, p, ip, ip, fp, NULL, 0, NULL), KARA_EHIP);
    EXPECT(kara_last_hip_error(), hipErrorLaunchFailure);
    EXPECT(kara_select_chunks(&c, fp, ip, bp, NULL), KARA_EHIP);
    EXPECT(kara_select_chunks_bridged(&c, 0, fp, ip, NULL, NULL), KARA_EHIP);
    EXPECT(kara_compact_paged(&c, p, p, ip, ip, ip, ip, ip, ip, NULL), KARA_EHIP);
    EXPECT(kara_compact_paged_tail(&c, p, p, ip, ip, ip, ip, ip, ip, ip, NULL), KARA_EHIP);
    EXPECT(kara_validate_tables(&c, ip, ip, ip, NULL), KARA_EHIP);
    EXPECT(kara_decode_attention(&c, p, p, p, ip, ip, fp, NULL, 0, NULL), KARA_EHIP);
    EXPECT(kara_compress_fused(&c, p, p, p, ip, ip, fp, ip, bp, ip, ip, ip, ip, NULL), KARA_EHIP);
    EXPECT(kara_compress_fused_noalloc(&c, p, p, p, ip, ip, fp, ip, bp, ip, ip, ip, NULL), KARA_EHIP);
    EXPECT(kara_last_hip_error(), hipErrorLaunchFailure);
    EXPECT(g_launches, calls + 1 + 1);   // nothing counted as launched
    g_fail_launch = 0;
  }
  for (int s = -8; s <= 2; ++s)
    if (!kara_status_str(s) || !strlen(kara_status_str(s))) ++fails;
  printf("host checks: %d launches, %d failures\n", g_launches, fails);
  return fails ? 1 : 0;
}
