// Host build of the kernels' segment walk (csrc/seg_walk.h): reads
// "B U L G n_0 ... n_{B-1}" on stdin, prints one line per segment:
// cta u t0 t1 host fin last iter0 n tok_off.
#include <cstdio>
#include <vector>

#define LA_HD
#include "seg_walk.h"

int main() {
    int B, U, L, G;
    if (std::scanf("%d %d %d %d", &B, &U, &L, &G) != 4) return 2;
    std::vector<int32_t> lens(B), tp(B + 1);
    std::vector<uint32_t> tok(B + 1);   // the kernels' width: up to 2^32 - 1 tokens in all
    for (int b = 0; b < B; ++b)
        if (std::scanf("%d", &lens[b]) != 1) return 2;
    tp[0] = 0;
    tok[0] = 0;
    for (int b = 0; b < B; ++b) {
        tp[b + 1] = tp[b] + (lens[b] + L - 1) / L;
        tok[b + 1] = tok[b] + lens[b];
    }
    for (int c = 0; c < G; ++c) {
        la::SegWalk<const int32_t*, const uint32_t*> w;
        w.init(tp.data(), tok.data(), B, U, G, c);
        la::LeanSeg s;
        while (w.next(s))
            std::printf("%d %d %d %d %d %d %d %d %d %lld\n", c, s.u, s.t0, s.t1, (int)s.host,
                        (int)s.fin, s.last, s.iter0, s.n, (long long)s.tok_off);
    }
    return 0;
}
