// Host-side check of the key-block partition shared by the state pass and the
// scan (state_block_frames, part_block_rows, part_block_subs in kernels.h) and
// of the state kernel's workgroup -> (block, sub-block) decode, for many
// geometries:
//  * the linear set each chunk reads is exactly the keys outside its softmax
//    window (recurrent form: the frames before max(t T_c - T_o, 0); the
//    bidirectional form: every frame outside [max(t T_c - T_o, 0),
//    min((t+1) T_c, F))), assembled from whole blocks;
//  * the backward's query blocks are the chunks' frames;
//  * sub-blocks cover each block's rows exactly, empty blocks have none;
//  * the decode of the launched workgroups hits every (block, sub-block) once.
// Built and run by tests/test_abi.py.
#include <cstdio>
#include <vector>

#include "kernels.h"

using namespace rehyat;

static int check_geometry(int mode, int F, int Tc, int To, int HW, int sub_rows) {
    int bad = 0;
    const int C = (F + Tc - 1) / Tc;
    const int U = state_block_count(mode, C);
    BlockPart part{mode, HW, Tc, To, F, 0, sub_rows};
    std::vector<int> f0(U), f1(U);
    for (int u = 0; u < U; ++u) {
        state_block_frames(mode, u, Tc, To, F, f0[u], f1[u]);
        int e0, e1;
        part_block_rows(part, u, e0, e1);
        if (e0 != f0[u] * HW || e1 != f1[u] * HW) ++bad;
        if (f0[u] < 0 || f0[u] > f1[u] || f1[u] > F) ++bad;
        if (u > 0 && f0[u] != f1[u - 1]) ++bad;  // blocks follow each other without gap or overlap
        const int n = part_block_subs(part, u), rows = e1 - e0;
        if (rows == 0 ? n != 0 : !((n - 1) * sub_rows < rows && rows <= n * sub_rows)) ++bad;
    }
    std::vector<char> in(F);
    if (mode == kCausal) {
        if (U > 0 && f0[0] != 0) ++bad;
        for (int t = 0; t < C; ++t) {  // linear set of chunk t = E_0 .. E_{t-1}
            for (int f = 0; f < F; ++f) in[f] = 0;
            for (int u = 0; u < t && u < U; ++u)
                for (int f = f0[u]; f < f1[u]; ++f) in[f] = 1;
            const int lin_end = t * Tc - To > 0 ? t * Tc - To : 0;
            for (int f = 0; f < F; ++f) bad += in[f] != (f < lin_end);
        }
    } else if (mode == kBidirectional) {
        if (f0[0] != 0 || f1[U - 1] != F) ++bad;
        const int q = To / Tc;
        for (int t = 0; t < C; ++t) {  // blocks before max(2(t - q), 0) and from 2t+3 on
            for (int f = 0; f < F; ++f) in[f] = 0;
            const int lo = 2 * (t - q) > 0 ? 2 * (t - q) : 0;
            for (int u = 0; u < U; ++u)
                if (u < lo || u >= 2 * t + 3)
                    for (int f = f0[u]; f < f1[u]; ++f) in[f] = 1;
            const int w0 = t * Tc - To > 0 ? t * Tc - To : 0, w1 = (t + 1) * Tc < F ? (t + 1) * Tc : F;
            for (int f = 0; f < F; ++f) bad += in[f] != (f < w0 || f >= w1);
        }
        for (int f = 0; f < F; ++f) {  // the block lookup by frame agrees with the ranges
            const int u = bidir_block_of_frame(f, Tc, To);
            if (u < 0 || u >= U || f < f0[u] || f >= f1[u]) ++bad;
        }
    } else {  // backward query blocks: chunk u + 1 (kChunkRows) or chunk u (kChunkRowsAll)
        for (int u = 0; u < U; ++u) {
            const int c = mode == kChunkRows ? u + 1 : u;
            if (f0[u] != c * Tc || f1[u] != ((c + 1) * Tc < F ? (c + 1) * Tc : F)) ++bad;
        }
    }
    // the state kernel's decode of its launched workgroups
    int items = 0;
    for (int u = 0; u < U; ++u) items += part_block_subs(part, u);
    std::vector<std::vector<int>> seen(U);
    for (int u = 0; u < U; ++u) seen[u].assign(part_block_subs(part, u), 0);
    for (int item = 0; item < items; ++item) {
        int sub = item, u = 0;
        for (; u < U - 1; ++u) {
            const int n = part_block_subs(part, u);
            if (sub < n) break;
            sub -= n;
        }
        if (sub < 0 || sub >= (int)seen[u].size()) { ++bad; continue; }
        ++seen[u][sub];
    }
    for (int u = 0; u < U; ++u)
        for (int s : seen[u]) bad += s != 1;
    return bad;
}

int main() {
    int bad = 0, cases = 0;
    for (int mode : {(int)kCausal, (int)kBidirectional, (int)kChunkRows, (int)kChunkRowsAll})
        for (int F : {1, 2, 3, 7, 21, 25})
            for (int Tc : {1, 2, 3, 7})
                for (int To : {0, 1, 2, 4, 5})
                    for (int HW : {16, 1560})
                        for (int sub_rows : {64, 1600, 1 << 20}) {
                            const int C = (F + Tc - 1) / Tc;
                            if (state_block_count(mode, C) <= 0) continue;
                            bad += check_geometry(mode, F, Tc, To, HW, sub_rows);
                            ++cases;
                        }
    printf("%d geometries, %d violations\n", cases, bad);
    return bad != 0;
}
