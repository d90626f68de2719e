// Host-only fuzz of the C-ABI argument validation: every entry point is called with fake
// (never dereferenced) pointers over random and extreme shapes, NULL, misaligned and
// overlapping arguments.  Built with the sanitizers against stand-in launchers (stubs.cpp);
// every return code must be a documented one.  Prints the number of calls that passed
// validation and the count of each return code.
#include <cstdio>
#include <cstdlib>
#include <random>
#include "gdn_verify.h"
extern int g_launches;
static std::mt19937_64 rng(1234);
static long long R(long long lo, long long hi) { return std::uniform_int_distribution<long long>(lo, hi)(rng); }
static float *F(long long slot) { return reinterpret_cast<float *>(0x7F0000000000ull + (unsigned long long)slot * (1ull << 34)); }
static const float *cf(long long s) { return F(s); }
static int32_t *I(long long s) { return reinterpret_cast<int32_t *>(F(s)); }
static void *maybe(void *p) { int r = (int)R(0, 40); if (r == 0) return nullptr; if (r == 1) return (char *)p + 4; if (r == 2) return (char *)p + 2; if (r == 3) return F(0); return p; }
static int widths[] = {16, 32, 64, 128, 24, 0, -16, 256};
static gdn_shape shape() {
    gdn_shape s;
    auto pick = [&](int a, int b) { return (int)R(a, b); };
    int mode = (int)R(0, 3);
    s.n_seqs = mode == 0 ? pick(-2, 2000) : pick(1, 1024);
    s.n_nodes = mode == 0 ? pick(-2, 70000) : (R(0, 1) ? pick(1, 32) : pick(1, 65536));
    s.n_slots = mode == 0 ? pick(-2, 1 << 26) : pick(1, 1 << 20);
    s.n_k_heads = mode == 0 ? pick(-1, 1 << 16) : pick(1, 64);
    s.n_v_heads = s.n_k_heads * (int)R(1, 4) + (mode == 0 ? (int)R(0, 1) : 0);
    s.d_k = widths[R(0, mode == 0 ? 7 : 3)];
    s.d_v = widths[R(0, mode == 0 ? 7 : 3)];
    s.d_conv = mode == 0 ? pick(0, 5) : 4;
    return s;
}
static bool known(int r) { return r >= 0 && r <= 8; }
int main() {
    int counts[9] = {0};
    for (int it = 0; it < 200000; ++it) {
        gdn_shape s = shape();
        const gdn_shape *sp = R(0, 50) ? &s : nullptr;
        long long b = R(1, 20);
        int which = (int)R(0, 9), r = 0;
        switch (which) {
        case 0: r = gdn_conv_tree_step(sp, cf(b), cf(b + 1), cf(b + 2), I(b + 3), I(b + 4), (int32_t *)maybe(I(b + 12)),
                                       (float *)maybe(F(b + 5)), (float *)maybe(F(b + 6)), (int32_t *)maybe(I(b + 7)), nullptr); break;
        case 1: r = gdn_tree_verify(sp, cf(b), cf(b + 1), cf(b + 2), R(-1, 200), cf(b + 3), cf(b + 4), cf(b + 5), I(b + 6),
                                    I(b + 7), (int32_t *)maybe(I(b + 12)), (float *)maybe(F(b + 8)), (float *)maybe(F(b + 9)),
                                    (int32_t *)maybe(I(b + 10)), nullptr); break;
        case 2: r = gdn_conv_tree_verify(sp, cf(b), cf(b + 1), cf(b + 2), cf(b + 3), cf(b + 4), R(-1, 200), cf(b + 5),
                                         cf(b + 6), cf(b + 7), I(b + 8), I(b + 9), (int32_t *)maybe(I(b + 12)),
                                         (float *)maybe(F(b + 10)), (float *)maybe(F(b + 11)), (float *)maybe(F(b + 13)),
                                         (int32_t *)maybe(I(b + 14)), nullptr); break;
        case 3: r = gdn_replay_commit(sp, cf(b), cf(b + 1), I(b + 2), I(b + 3), (int32_t *)maybe(I(b + 12)), I(b + 4),
                                      (float *)maybe(F(b + 5)), (float *)maybe(F(b + 6)), (int32_t *)maybe(I(b + 7)), nullptr); break;
        case 4: {
            int L = (int)R(-1, 70);
            const float *logs[80], *wins[80]; float *pools[80], *hists[80];
            for (int l = 0; l < 80; ++l) { logs[l] = cf(b + 20 + 4 * l); wins[l] = cf(b + 21 + 4 * l); pools[l] = F(b + 22 + 4 * l); hists[l] = F(b + 23 + 4 * l); }
            if (R(0, 5) == 0) pools[R(0, 79)] = pools[0];
            r = gdn_replay_commit_layers(sp, L, R(0, 30) ? logs : nullptr, wins, I(b + 2), I(b + 3), (int32_t *)maybe(I(b + 12)),
                                         I(b + 4), pools, hists, (int32_t *)maybe(I(b + 7)), nullptr); break;
        }
        case 5: r = gdn_conv_step(sp, cf(b), cf(b + 1), (float *)maybe(F(b + 2)), I(b + 3), (float *)maybe(F(b + 4)),
                                  (int32_t *)maybe(I(b + 5)), nullptr); break;
        case 6: r = gdn_decode_step(sp, cf(b), cf(b + 1), cf(b + 2), R(-1, 200), cf(b + 3), cf(b + 4), (float *)maybe(F(b + 5)),
                                    I(b + 6), (float *)maybe(F(b + 7)), (int32_t *)maybe(I(b + 8)), nullptr); break;
        case 7: {
            size_t need = gdn_prefill_workspace_size(sp);
            size_t have = R(0, 3) ? need : (size_t)R(0, 1 << 30);
            r = gdn_prefill(sp, cf(b), cf(b + 1), cf(b + 2), R(-1, 200), cf(b + 3), cf(b + 4), (float *)maybe(F(b + 5)),
                            I(b + 6), R(0, 1) ? cf(b + 7) : nullptr, (int32_t)R(-1, 2), (float *)maybe(F(b + 8)),
                            (float *)maybe(F(b + 9)), have, (int32_t *)maybe(I(b + 10)), nullptr); break;
        }
        case 8: r = gdn_prefill_noalloc(sp, cf(b), cf(b + 1), cf(b + 2), R(-1, 200), cf(b + 3), cf(b + 4),
                                        (float *)maybe(F(b + 5)), I(b + 6), R(0, 1) ? cf(b + 7) : nullptr,
                                        (int32_t)R(-1, 2), (float *)maybe(F(b + 8)), (int32_t *)maybe(I(b + 10)),
                                        nullptr); break;
        case 9: r = gdn_conv_decode_step(sp, cf(b), cf(b + 1), (float *)maybe(F(b + 2)), cf(b + 3), cf(b + 4), R(-1, 200),
                                         cf(b + 5), cf(b + 6), (float *)maybe(F(b + 7)), I(b + 8),
                                         (int32_t *)maybe(I(b + 9)), (float *)maybe(F(b + 10)),
                                         (int32_t *)maybe(I(b + 11)), nullptr); break;
        }
        if (!known(r)) { std::printf("unknown return %d from call %d\n", r, which); return 1; }
        ++counts[r];
        if (!gdn_strerror(r)) return 1;
    }
    std::printf("launches %d; codes:", g_launches);
    for (int k = 0; k < 9; ++k) std::printf(" %d:%d", k, counts[k]);
    std::printf("\n");
    return 0;
}
