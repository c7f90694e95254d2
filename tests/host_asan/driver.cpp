// Drives the C ABI's ring bookkeeping on a bookkeeping-only cache from a
// command list on stdin, printing the return code and the visible-page
// list after every command (compared with the oracle by the test).
//   C P W nfpb S cross ns R maxf   create (replacing any previous cache)
//   A t keyframe                   kvcache_append on layer 0 (and layer 1)
//   E | R | X                      evict | rollback | reset
// Argument-error calls are made once at the start.
#include <cstdio>
#include <cstring>
#include <vector>

#include "swa.h"

static void pages(swa_cache* c, int layer) {
    int n = 0;
    kvcache_visible_pages(c, layer, nullptr, 0, &n);
    std::vector<swa_page> buf(n > 0 ? n : 1);
    kvcache_visible_pages(c, layer, buf.data(), n, &n);
    std::printf("P %d", n);
    for (int i = 0; i < n; ++i)
        std::printf(" %d %d %d %d %d", buf[i].frame, buf[i].region, buf[i].slot, buf[i].row0, buf[i].nrows);
    std::printf("\n");
}

int main() {
    // error paths that need no device
    swa_config bad{};
    std::printf("E0 %d %zu\n", swa_cache_create(&bad, nullptr, 0, nullptr), swa_cache_pool_bytes(&bad));
    std::printf("E1 %d\n", swa_graph_step(nullptr, 0, 1, nullptr));
    std::printf("E2 %zu %zu\n", swa_decode_cache_bytes(0, 8, 4096, 64), swa_decode_workspace_bytes(32, 5, 64));
    swa_cache* c = nullptr;
    char op[8];
    while (std::scanf("%7s", op) == 1) {
        int rc = 0;
        if (!std::strcmp(op, "C")) {
            swa_config cfg{};
            int P, W, nfpb, S, cross, ns, R, maxf;
            if (std::scanf("%d %d %d %d %d %d %d %d", &P, &W, &nfpb, &S, &cross, &ns, &R, &maxf) != 8) return 2;
            cfg.num_layers = 2;
            cfg.tokens_per_frame = P;
            cfg.num_heads = 2;
            cfg.head_dim = 64;
            cfg.dtype = SWA_BF16;
            cfg.sliding_window_size = W;
            cfg.num_frame_per_block = nfpb;
            cfg.scale_frames = S;
            cfg.cross_frame_special = cross;
            cfg.special_row0 = 0;
            cfg.special_rows = ns;
            cfg.max_special_frames = R;
            cfg.max_frames = maxf;
            if (c != nullptr) swa_cache_destroy(c);
            c = nullptr;
            rc = swa_cache_create(&cfg, nullptr, 0, &c);
            swa_graph* g = nullptr;
            std::printf("G %d\n", swa_graph_create(c, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                                   0.f, &g));
        } else if (!std::strcmp(op, "A")) {
            long long t;
            int kf;
            if (std::scanf("%lld %d", &t, &kf) != 2) return 2;
            rc = kvcache_append(c, 0, t, nullptr, nullptr, kf, nullptr);
            kvcache_append(c, 1, t, nullptr, nullptr, kf, nullptr);
        } else if (!std::strcmp(op, "E")) {
            rc = kvcache_evict(c, 0, nullptr);
            kvcache_evict(c, 1, nullptr);
        } else if (!std::strcmp(op, "R")) {
            rc = kvcache_rollback(c, 0, nullptr);
            kvcache_rollback(c, 1, nullptr);
        } else if (!std::strcmp(op, "X")) {
            rc = kvcache_reset(c, nullptr);
        } else {
            return 2;
        }
        std::printf("%s %d\n", op, rc);
        if (c != nullptr) pages(c, 1);
    }
    if (c != nullptr) swa_cache_destroy(c);
    return 0;
}
