// CPU check of the index maps used by the block-sparse attention kernel:
// bijections, bounds, the MFMA k-slot relabelling, and an LDS bank model of
// the V^T staging writes and operand reads.  Runs on the host only.
#include <stdio.h>
#include <stdlib.h>

#include <set>
#include <vector>

#include "attn_layout.hpp"

static int failures = 0;
#define CHECK(cond, ...)                    \
    do {                                    \
        if (!(cond)) {                      \
            printf("FAIL: " __VA_ARGS__);   \
            printf("\n");                   \
            ++failures;                     \
        }                                   \
    } while (0)

// Max number of distinct addresses (4-byte words) falling in one bank, over
// the lanes serviced together.
static int bank_ways(const std::vector<int>& byte_addr, const std::vector<int>& bytes, int banks) {
    std::vector<std::set<int>> words(banks);
    for (size_t i = 0; i < byte_addr.size(); ++i)
        for (int b = 0; b < bytes[i]; b += 4) {
            const int w = (byte_addr[i] + b) / 4;
            words[w % banks].insert(w);
        }
    int worst = 0;
    for (auto& s : words) worst = s.size() > (size_t)worst ? (int)s.size() : worst;
    return worst;
}

template <int D>
static void check_d() {
    constexpr int CH = D / 8;
    // tok_pos: bijection within each 16-token group, and the k-slot relabelling
    std::set<int> seen;
    for (int t = 0; t < 64; ++t) {
        const int p = vsa::tok_pos(t);
        CHECK(p >= 0 && p < 64 && p / 16 == t / 16, "tok_pos(%d)=%d", t, p);
        seen.insert(p);
    }
    CHECK(seen.size() == 64, "tok_pos not a bijection");
    for (int s4 = 0; s4 < 4; ++s4)
        for (int hh = 0; hh < 2; ++hh)
            for (int jj = 0; jj < 2; ++jj)
                for (int ii = 0; ii < 4; ++ii)
                    CHECK(vsa::tok_pos(16 * s4 + 8 * jj + 4 * hh + ii) == 16 * s4 + 8 * hh + 4 * jj + ii,
                          "k-slot relabelling s4=%d hh=%d jj=%d ii=%d", s4, hh, jj, ii);
    // vt_off: bijection onto [0, D*64)
    std::vector<int> hit(D * 64, 0);
    for (int d = 0; d < D; ++d)
        for (int p = 0; p < 64; ++p) {
            const int o = vsa::vt_off(d, p);
            CHECK(o >= 0 && o < D * 64, "vt_off(%d,%d)=%d out of range", d, p, o);
            if (o >= 0 && o < D * 64) hit[o]++;
        }
    for (int o = 0; o < D * 64; ++o) CHECK(hit[o] == 1, "vt_off hits %d %d times", o, hit[o]);
    // staging units cover every (g4, c) once
    std::vector<int> cov(16 * CH, 0);
    for (int u = 0; u < 16 * CH; ++u) {
        int g4, c;
        vsa::stage_unit<CH>(u, &g4, &c);
        CHECK(g4 >= 0 && g4 < 16 && c >= 0 && c < CH, "unit %d -> (%d,%d)", u, g4, c);
        cov[g4 * CH + c]++;
    }
    for (int x = 0; x < 16 * CH; ++x) CHECK(cov[x] == 1, "unit coverage %d = %d", x, cov[x]);

    // bank model, 32 banks x 4 bytes: ds_write_b64 serviced 16 lanes at a time
    int worst_w = 0;
    for (int wave_instr = 0; wave_instr < 16 * CH / 64; ++wave_instr)
        for (int e = 0; e < 8; ++e)
            for (int quarter = 0; quarter < 4; ++quarter) {
                std::vector<int> a, b;
                for (int l = 16 * quarter; l < 16 * quarter + 16; ++l) {
                    int g4, c;
                    vsa::stage_unit<CH>(64 * wave_instr + l, &g4, &c);
                    a.push_back(2 * vsa::vt_off(8 * c + e, vsa::tok_pos(4 * g4)));
                    b.push_back(8);
                }
                const int w = bank_ways(a, b, 32);
                worst_w = w > worst_w ? w : worst_w;
            }
    // ds_read_b128 of the V^T operand serviced 8 lanes at a time
    int worst_r = 0;
    for (int dt = 0; dt < D / 32; ++dt)
        for (int s4 = 0; s4 < 4; ++s4)
            for (int oct = 0; oct < 8; ++oct) {
                std::vector<int> a, b;
                for (int l = 8 * oct; l < 8 * oct + 8; ++l) {
                    const int d = 32 * dt + (l & 31), hh = l >> 5;
                    a.push_back(2 * vsa::vt_off(d, 16 * s4 + 8 * hh));
                    b.push_back(16);
                }
                const int w = bank_ways(a, b, 32);
                worst_r = w > worst_r ? w : worst_r;
            }
    printf("D=%d: worst bank ways (32x4B model): staging write %d, operand read %d\n", D, worst_w, worst_r);
    CHECK(worst_w == 1, "staging writes conflict (%d-way)", worst_w);
    CHECK(worst_r == 1, "operand reads conflict (%d-way)", worst_r);
}

int main() {
    check_d<128>();
    check_d<64>();
    // xcd_remap is a bijection of [0, N)
    const int Ns[] = {1, 2, 7, 8, 9, 15, 16, 17, 63, 64, 65, 242, 1000, 13552, 16896, 100003};
    for (int N : Ns) {
        std::vector<char> hit(N, 0);
        for (int n = 0; n < N; ++n) {
            const int m = vsa::xcd_remap(n, N);
            CHECK(m >= 0 && m < N, "xcd_remap(%d,%d)=%d", n, N, m);
            if (m >= 0 && m < N) hit[m]++;
        }
        for (int m = 0; m < N; ++m) CHECK(hit[m] == 1, "xcd_remap N=%d misses %d", N, m);
    }
    if (failures) {
        printf("%d failures\n", failures);
        return 1;
    }
    printf("layout checks passed\n");
    return 0;
}
