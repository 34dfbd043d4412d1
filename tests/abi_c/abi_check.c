/*
 * A plain C11 caller of libkvevict: include/kvevict.h must compile as C and
 * the library must link and answer from C.  Only host entry points and the
 * device entry points' argument validation are exercised (no GPU needed):
 * every device call below is refused before anything is enqueued.  Prints one
 * "name value" line per check; the Python test compares them.
 */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "kvevict.h"

static void show(const char *name, int rc) {
    printf("%s %d\n", name, rc);
}

int main(int argc, char **argv) {
    if (argc != 2) return 2;
    const kvx_shape sh = {28, 1, 8, 128, KVX_BF16};
    kvx_evict_params p = {4096, 4, 0, KVX_KEEP_LOW};
    size_t ws = 1;
    show("abi_version", kvx_abi_version());
    show("workspace_rc", kv_evict_workspace_size(sh, 4096, 4096, p, &ws));
    printf("workspace_onchip %zu\n", ws);
    kvx_evict_params big = {1 << 20, 4, 0, KVX_KEEP_HIGH};
    kv_evict_workspace_size(sh, 1 << 20, 1 << 20, big, &ws);
    printf("workspace_multiblock %zu\n", ws);

    /* validation before launch: every pointer below is bogus and never read */
    float dummy[4];
    int32_t idx[4];
    kvx_evict_params bad = {4096, 4096, 0, KVX_KEEP_LOW};
    show("topk_bad_params", kv_evict_topk(dummy, dummy, sh, 4096, 4096, bad, idx, NULL, 0, NULL));
    show("topk_null_idx", kv_evict_topk(dummy, dummy, sh, 4096, 4096, p, NULL, NULL, 0, NULL));
    show("score_bad_mode", qf_score_keys(dummy, sh, 16, 7, NULL, 1, dummy, NULL));
    show("score_proj_no_filters", qf_score_keys(dummy, sh, 16, KVX_SCORE_PROJ, NULL, 1, dummy, NULL));
    kvx_shape bad_d = sh;
    bad_d.D = 96;
    show("score_bad_head_dim", qf_score_keys(dummy, bad_d, 16, KVX_SCORE_L2, NULL, 1, dummy, NULL));
    show("gather_partial_alias", kv_compact_gather(dummy, dummy, dummy, idx, dummy, dummy, dummy, 0, idx, sh, 100, 10,
                                                   p, dummy, (void *)idx, dummy, idx, NULL));
    show("decode_position_range", kv_evict_one_inplace(dummy, dummy, dummy, idx, dummy, dummy, dummy,
                                                       (int64_t)1 << 40, sh, 4096, p, NULL));
    char msg[256];
    snprintf(msg, sizeof msg, "%s", kvx_last_error());
    printf("last_error_mentions_int32 %d\n", strstr(msg, "int32") != NULL);

    /* host entry points */
    float f[2 * 2 * 4];
    for (int i = 0; i < 16; ++i) f[i] = (float)(i % 5) - 1.5f;
    show("save", qf_filters_save(argv[1], f, 2, 2, 4, "org/model", 7, "synthetic"));
    float g[16];
    int64_t n_samples = 0;
    show("load", qf_filters_load(argv[1], "org/model", 2, 2, 4, g, &n_samples));
    printf("load_same %d\n", memcmp(f, g, sizeof f) == 0 && n_samples == 7);
    show("load_other_model", qf_filters_load(argv[1], "org/other", 2, 2, 4, g, NULL));
    show("load_missing_layer", qf_filters_load(argv[1], NULL, 3, 2, 4, g, NULL));

    float q[2 * 16 * 4], out[4];
    for (int h = 0; h < 2; ++h)
        for (int r = 0; r < 16; ++r)
            for (int d = 0; d < 4; ++d) q[(h * 16 + r) * 4 + d] = (d == 1 ? 2.0f + 0.1f * (float)r : 0.0f) +
                                                                 0.01f * (float)((h + r * 3 + d * 7) % 5);
    show("from_queries", qf_filters_from_queries(q, 2, 16, 4, 1, out));
    printf("from_queries_unit %d\n", fabs(out[0] * out[0] + out[1] * out[1] + out[2] * out[2] + out[3] * out[3] - 1.0) < 1e-6);
    printf("from_queries_axis %d\n", out[1] > 0.99f);

    kvx_stats_t st;
    show("stats", kvx_stats(sh, 32768, 4096, KVX_SCORE_PROJ, &st));
    printf("stats_ratio %.1f\n", st.compression_ratio);
    return 0;
}
