// CPU check of the index maps used by the block-sparse attention kernel.
// It simulates, on the host, the direct global->LDS copies of one K and one V
// block into their swizzled tiles and every MFMA operand fetch from them
// (ds_read_b128 for K, ds_read_b64_tr_b16 for V, the latter with the lane
// rule of the hardware: within a 16-lane group, lane i receives element i & 3
// of the 8-byte chunks addressed by lanes (i >> 2) + 4 r, r = 0..3), and
// checks that every lane gets exactly the K / V elements the MFMA layout
// needs.  Also: bounds, bijections, an LDS bank model, the XCD remap.
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <set>
#include <vector>

#include "attn_layout.hpp"
#include "vsa_internal.hpp"

static int failures = 0;
#define CHECK(cond, ...)                  \
    do {                                  \
        if (!(cond)) {                    \
            if (failures < 20) {          \
                printf("FAIL: " __VA_ARGS__); \
                printf("\n");             \
            }                             \
            ++failures;                   \
        }                                 \
    } while (0)

// Max number of distinct 4-byte words falling in one bank over the lanes
// serviced together.
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

// value stored for element (token t, dim d) of a block: unique and recognisable
static int val(int t, int d) { return t * 1000 + d; }

template <int D, int SW>
static std::vector<int> fill_tile(int valid) {
    constexpr int CH = D / 8;
    constexpr int ROWB = CH * 16;  // bytes per source row
    std::vector<int> tile(64 * D, -1);
    std::vector<int> hits(64 * CH, 0);
    for (int wave = 0; wave < 2; ++wave)
        for (int n = 0; n < CH / 2; ++n)
            for (int lane = 0; lane < 64; ++lane) {
                const int p = vsa::load_chunk_pos(n, wave, lane);
                CHECK(p >= 0 && p < 64 * CH, "chunk position %d out of range", p);
                hits[p]++;
                const int row = p / CH;
                const int sw = vsa::tile_swz<CH, SW>(row);
                const int c = (p % CH) ^ sw;
                CHECK(c >= 0 && c < CH, "logical chunk %d out of range", c);
                // full blocks use the fixed per-lane offset of n & 1 + 4096 (n >> 1)
                const int fast = vsa::lane_src_offset<CH, SW>(wave, lane, n & 1) + 4096 * (n >> 1);
                CHECK(fast == row * ROWB + 16 * c, "fast-path offset D%d SW%d n%d w%d l%d", D, SW, n, wave, lane);
                CHECK(fast >= 0 && fast + 16 <= 64 * ROWB, "fast-path offset out of the block");
                const int src_row = row < valid ? row : valid - 1;
                const int src_byte = valid == 64 ? fast : src_row * ROWB + 16 * c;
                CHECK(src_byte / ROWB < valid, "copy reads past the valid rows");
                // lane's 16 bytes land at byte 16*lane of the wave's 1 KiB segment
                const int lds_elem = (2 * n + wave) * 64 * 8 + 8 * lane;
                CHECK(lds_elem == 8 * p, "segment placement");
                for (int e = 0; e < 8; ++e) tile[lds_elem + e] = val(src_byte / ROWB, (src_byte % ROWB) / 2 + e);
            }
    for (int p = 0; p < 64 * CH; ++p) CHECK(hits[p] == 1, "chunk %d written %d times", p, hits[p]);
    return tile;
}

// The NW-wave copy (load_tile_n, NW = 4 or 8): every chunk written once, the
// fast-path lane offset plus 1024 NW n equals the per-instruction one, partial
// or strided blocks (rows PITCH bytes apart) clamp inside the valid rows and
// read inside each row, and the resulting tile equals the two-wave one.
template <int D, int SW, int ROWS = 64, int NW = 4>
static std::vector<int> fill_tileN(int valid, int pitch = D * 2) {
    constexpr int CH = D / 8;
    constexpr int ROWB = CH * 16;
    constexpr int RSTEP = 64 * NW / CH;
    constexpr int NI = ROWS * CH / (64 * NW);
    static_assert(NI >= 1 && NI * 64 * NW == ROWS * CH, "whole instructions");
    std::vector<int> tile(ROWS * D, -1);
    std::vector<int> hits(ROWS * CH, 0);
    for (int wave = 0; wave < NW; ++wave)
        for (int n = 0; n < NI; ++n)
            for (int lane = 0; lane < 64; ++lane) {
                const int p = vsa::load_chunk_posN<NW>(n, wave, lane);
                CHECK(p >= 0 && p < ROWS * CH, "chunk position %d out of range (%d waves)", p, NW);
                hits[p]++;
                const int row = p / CH;
                const int c = (p % CH) ^ vsa::tile_swz<CH, SW>(row);
                const int fast = vsa::lane_src_offsetN<CH, SW, NW>(wave, lane) + 1024 * NW * n;
                CHECK(fast == row * ROWB + 16 * c, "%d-wave fast-path offset D%d SW%d n%d w%d l%d", NW, D, SW, n,
                      wave, lane);
                // the kernel's partial-block formula
                const int p0 = vsa::load_chunk_posN<NW>(0, wave, lane);
                const int row0 = p0 / CH;
                const int c0 = (p0 % CH) ^ vsa::tile_swz<CH, SW>(row0);
                const int rk = std::min(row0, valid - 1 - RSTEP * n) + RSTEP * n;
                CHECK(row0 + RSTEP * n == row && c0 == c, "%d-wave partial-path row/chunk", NW);
                CHECK(rk == std::min(row, valid - 1), "%d-wave partial-path clamp", NW);
                // byte offset in the source block of rows `pitch` bytes apart
                const bool fast_path = valid >= ROWS && pitch == ROWB;
                const long src = fast_path ? fast : (long)rk * pitch + 16 * c0;
                CHECK(src / pitch < valid && src % pitch + 16 <= ROWB, "%d-wave copy reads outside the valid rows", NW);
                const int srow = (int)(src / pitch), sbyte = (int)(src % pitch);
                const int lds_elem = (NW * n + wave) * 64 * 8 + 8 * lane;
                for (int e = 0; e < 8; ++e) tile[lds_elem + e] = val(srow, sbyte / 2 + e);
            }
    for (int p = 0; p < ROWS * CH; ++p) CHECK(hits[p] == 1, "chunk %d written %d times (%d waves)", p, hits[p], NW);
    return tile;
}

template <int D, int SW, int ROWS = 64>
static std::vector<int> fill_tile4(int valid) {
    return fill_tileN<D, SW, ROWS, 4>(valid);
}

// Row operand (the A operand of S^T = K Q^T, or of S = Q K^T / dP = dO V^T in
// the backward): lane l gets T[32 mt + l%32][16 ks + 8 hh + 0..7].
template <int D, int SW>
static void check_row_operand(const std::vector<int>& t, int valid) {
    constexpr int CH = D / 8, KS = D / 16;
    for (int mt = 0; mt < 2; ++mt)
        for (int ks = 0; ks < KS; ++ks)
            for (int l = 0; l < 64; ++l) {
                const int row = 32 * mt + (l & 31), hh = l >> 5;
                const int off = vsa::tile_off<CH>(row, 2 * ks + hh, vsa::tile_swz<CH, SW>(row));
                const int r = row < valid ? row : valid - 1;
                for (int e = 0; e < 8; ++e)
                    CHECK(t[off + e] == val(r, 16 * ks + 8 * hh + e), "row operand SW%d mt%d ks%d lane%d e%d", SW, mt,
                          ks, l, e);
            }
}

// Transposed operand (V^T of O^T = V^T P^T; K^T, Q^T, dO^T in the backward)
// via two transpose reads per k-step: lane l needs T[16 s4 + 8 jj + 4 hh +
// r][32 dt + l%32] in slot 4 jj + r.
template <int D, int SW>
static void tr_addresses(int dt, int s4, int jj, int* addr) {
    constexpr int CH = D / 8;
    for (int l = 0; l < 64; ++l) {
        const int g16 = l >> 4, L16 = l & 15, hh = l >> 5;
        const int tok = 16 * s4 + 8 * jj + 4 * hh + vsa::tr_token(L16);
        const int d = 32 * dt + 16 * (g16 & 1) + 4 * vsa::tr_dquad(L16);
        addr[l] = vsa::tile_off<CH>(tok, d >> 3, vsa::tile_swz<CH, SW>(tok)) + (d & 7);
    }
}
template <int D, int SW>
static void check_tr_operand(const std::vector<int>& t, int valid) {
    constexpr int DT = D / 32;
    for (int dt = 0; dt < DT; ++dt)
        for (int s4 = 0; s4 < 4; ++s4)
            for (int jj = 0; jj < 2; ++jj) {
                int addr[64];
                tr_addresses<D, SW>(dt, s4, jj, addr);
                for (int l = 0; l < 64; ++l) CHECK(addr[l] >= 0 && addr[l] + 3 < 64 * D, "tr address out of range");
                for (int l = 0; l < 64; ++l) {
                    const int grp = l & ~15, i = l & 15, hh = l >> 5;
                    for (int r = 0; r < 4; ++r) {
                        const int src = grp + (i >> 2) + 4 * r;
                        const int got = t[addr[src] + (i & 3)];
                        const int tok = 16 * s4 + 8 * jj + 4 * hh + r;
                        const int tt = tok < valid ? tok : valid - 1;
                        CHECK(got == val(tt, 32 * dt + (l & 31)), "tr operand SW%d dt%d s4%d jj%d lane%d r%d", SW, dt,
                              s4, jj, l, r);
                    }
                }
            }
}

// LDS bank model: worst ways of the row reads (b128) and of the transpose
// reads (b64) of a tile, with `banks` banks of 4 bytes (passes of 4 banks
// bytes).
template <int D, int SW>
static int bank_row(int banks) {
    constexpr int CH = D / 8, KS = D / 16;
    int worst = 0;
    for (int mt = 0; mt < 2; ++mt)
        for (int ks = 0; ks < KS; ++ks) {
            const int lpp = banks * 4 / 16;
            for (int p0 = 0; p0 < 64; p0 += lpp) {
                std::vector<int> a, b;
                for (int l = p0; l < p0 + lpp; ++l) {
                    const int row = 32 * mt + (l & 31);
                    a.push_back(2 * vsa::tile_off<CH>(row, 2 * ks + (l >> 5), vsa::tile_swz<CH, SW>(row)));
                    b.push_back(16);
                }
                const int w = bank_ways(a, b, banks);
                worst = w > worst ? w : worst;
            }
        }
    return worst;
}
template <int D, int SW>
static int bank_tr(int banks) {
    constexpr int DT = D / 32;
    int worst = 0;
    for (int dt = 0; dt < DT; ++dt)
        for (int s4 = 0; s4 < 4; ++s4)
            for (int jj = 0; jj < 2; ++jj) {
                int addr[64];
                tr_addresses<D, SW>(dt, s4, jj, addr);
                const int lpp = banks * 4 / 8;
                for (int p0 = 0; p0 < 64; p0 += lpp) {
                    std::vector<int> a, b;
                    for (int l = p0; l < p0 + lpp; ++l) {
                        a.push_back(2 * addr[l]);
                        b.push_back(8);
                    }
                    const int w = bank_ways(a, b, banks);
                    worst = w > worst ? w : worst;
                }
            }
    return worst;
}

template <int D>
static void check_d() {
    constexpr int CH = D / 8;
    // swizzles are permutations of a row's chunks
    for (int row = 0; row < 64; ++row) {
        std::set<int> a, b, c;
        for (int x = 0; x < CH; ++x) {
            a.insert(vsa::tile_off<CH>(row, x, vsa::k_swz<CH>(row)));
            b.insert(vsa::tile_off<CH>(row, x, vsa::v_swz<CH>(row)));
            c.insert(vsa::tile_off<CH>(row, x, vsa::dual_swz<CH>(row)));
        }
        CHECK((int)a.size() == CH && (int)b.size() == CH && (int)c.size() == CH,
              "swizzle of row %d not a permutation", row);
        CHECK(*a.rbegin() < 64 * D && *b.rbegin() < 64 * D && *c.rbegin() < 64 * D, "tile offset out of range");
    }
    for (int valid : {64, 37, 1}) {
        check_row_operand<D, vsa::kSwzRow>(fill_tile<D, vsa::kSwzRow>(valid), valid);
        check_tr_operand<D, vsa::kSwzTr>(fill_tile<D, vsa::kSwzTr>(valid), valid);
        const std::vector<int> dual = fill_tile<D, vsa::kSwzDual>(valid);
        check_row_operand<D, vsa::kSwzDual>(dual, valid);
        check_tr_operand<D, vsa::kSwzDual>(dual, valid);
        const bool same4 = fill_tile4<D, vsa::kSwzDual>(valid) == dual;
        CHECK(same4, "4-wave copy differs from the 2-wave one (D=%d)", D);
        // a 32-row tile: the first 32 rows of the 64-row layout (rows clamped
        // to min(valid, 32) - 1), read by the same row and transposed operands
        const int v32 = valid < 32 ? valid : 32;
        const std::vector<int> half = fill_tile4<D, vsa::kSwzDual, 32>(v32);
        const std::vector<int> ref32 = fill_tile<D, vsa::kSwzDual>(v32);
        const bool same32 = std::equal(half.begin(), half.end(), ref32.begin());
        CHECK(same32, "32-row 4-wave copy differs from the first rows of the 64-row layout (D=%d)", D);
        // the forward's K (row) and V (transposed) tiles copied by the 4 or 8
        // waves of a workgroup that serves 2 or 4 query blocks, with rows
        // contiguous or 2*D*H bytes apart ([B,S,H,D] with H = 3)
        for (int pitch : {2 * D, 2 * D * 3}) {
            const std::vector<int> k2 = fill_tile<D, vsa::kSwzRow>(valid);
            const std::vector<int> v2 = fill_tile<D, vsa::kSwzTr>(valid);
            CHECK((fill_tileN<D, vsa::kSwzRow, 64, 4>(valid, pitch) == k2), "4-wave K tile (D=%d pitch %d)", D, pitch);
            CHECK((fill_tileN<D, vsa::kSwzTr, 64, 4>(valid, pitch) == v2), "4-wave V tile (D=%d pitch %d)", D, pitch);
            CHECK((fill_tileN<D, vsa::kSwzRow, 64, 8>(valid, pitch) == k2), "8-wave K tile (D=%d pitch %d)", D, pitch);
            CHECK((fill_tileN<D, vsa::kSwzTr, 64, 8>(valid, pitch) == v2), "8-wave V tile (D=%d pitch %d)", D, pitch);
        }
    }
    for (int banks : {32, 64}) {
        const int kr = bank_row<D, vsa::kSwzRow>(banks), vt = bank_tr<D, vsa::kSwzTr>(banks);
        const int dr = bank_row<D, vsa::kSwzDual>(banks), dtr = bank_tr<D, vsa::kSwzDual>(banks);
        printf("D=%d, %d banks: worst ways K rows %d, V transposed %d, dual rows %d, dual transposed %d\n", D, banks,
               kr, vt, dr, dtr);
        // the forward's K and V tiles are conflict-free with 32 banks (and with
        // 64 for D = 128); the dual layout is made for gfx950's 64 banks
        if (banks == 32 || D == 128) CHECK(kr == 1 && vt == 1, "bank conflicts (D=%d, %d banks)", D, banks);
        if (banks == 64) CHECK(dr == 1 && dtr == 1, "dual layout bank conflicts (D=%d)", D);
    }
}

// Operand reads of the float64 MFMA block-level products (v_mfma_f64_16x16x4):
// lane (m = lane % 16, g = lane / 16) reads element m of staged row g, rows
// `pitch` doubles apart (64 or 32 values plus 16 of padding).  Each half-wave
// of a ds_read_b64 (32 lanes, two rows) must touch 64 distinct banks; without
// the padding the two rows of a half-wave share their banks.
static void check_f64_mfma_operands() {
    const int rows[] = {64, 32};
    for (int len : rows) {
        for (int pad : {16, 0}) {
            const int pitch = len + pad;
            int worst = 0;
            for (int col0 = 0; col0 + 16 <= len; col0 += 16)
                for (int half = 0; half < 2; ++half) {
                    std::vector<int> addr, bytes;
                    for (int l = 32 * half; l < 32 * half + 32; ++l) {
                        addr.push_back(8 * ((l / 16) * pitch + col0 + l % 16));
                        bytes.push_back(8);
                    }
                    const int w = bank_ways(addr, bytes, 64);
                    worst = w > worst ? w : worst;
                }
            if (pad) CHECK(worst == 1, "f64 MFMA operand reads conflict (row %d, pitch %d)", len, pitch);
            else CHECK(worst == 2, "unpadded rows expected two-way (row %d)", len);
        }
    }
}

int main() {
    check_d<128>();
    check_d<64>();
    check_f64_mfma_operands();
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
