// bwd.hip -- backward of the ReHyAt hybrid attention (recurrent partition).
//
// Forward (arXiv 2601.04342, §3.1-§3.3): for query i of chunk t,
//   y_i = (sum_{j in T^S_t} e^{q_i.k_j} v_j + sum_{j in T^L_t} (phi(q_i).phi(k_j)) v_j) / N_i,
// N_i = n^S_i + n^L_i, lse_i = ln N_i.  With the weights w_ij (e^{q.k} on the
// softmax set, phi(q).phi(k) on the linear set), D_i = dy_i . y_i and the
// normalised weights w_ij / N_i:
//   dv_j      = sum_i (w_ij / N_i) dy_i
//   dw_ij     = (dy_i . v_j - D_i) / N_i
//   softmax:  ds_ij = (w_ij / N_i)(dy_i . v_j - D_i);  dq_i += ds_ij k_j,  dk_j += ds_ij q_i
//   linear:   dphi(q_i) = e^{-lse_i} (S_t dy_i - D_i z_t)          (S_t = sum_{T^L_t} phi(k) v^T)
//             dphi(k_j) = G_u v_j - g_u,  dv_j += G_u^T phi(k_j)   (j in delta block E_u)
//             G_u = sum_{t > u} sum_{i in chunk t} e^{-lse_i} phi(q_i) dy_i^T,
//             g_u = sum_{t > u} sum_{i in chunk t} e^{-lse_i} D_i phi(q_i)
//   dq_i += phi'(q_i) . dphi(q_i),  dk_j += phi'(k_j) . dphi(k_j)   (elementwise maps)
// The G_u are the reverse-order (suffix) counterpart of the forward's state
// scan; they come from the block-state kernel run over query rows with dy as
// its second operand, and a suffix scan.
//
// bf16 kernels, both on v_mfma_f32_32x32x16_bf16 with fp32 accumulation:
//  * dk/dv: a workgroup of 8 waves owns 128 keys and streams the query rows of
//    the chunks whose windows hold them (64-row Q and dY tiles in a 3-stage LDS
//    ring, with each row's lse, D and window bounds).  Two waves share 32 keys
//    (one per lane): the first holds their K fragments and forms S = Q K^T, P
//    and dV^T += dY^T P, and passes P (bf16) through LDS to the second, which
//    holds V, runs one tile behind and forms dP = dY V^T, dS = P (dP - D) and
//    dK^T += Q^T dS.  dY^T and Q^T come through the transposing LDS read in the
//    key order of P's registers.  The linear branch of the keys is added first
//    from G_u (both layouts, bf16 hi/lo) and g_u.
//  * dq: a workgroup of 8 waves owns 256 queries of one chunk (q and dy
//    fragments in registers) and streams its window's K and V tiles (64 keys,
//    2-stage ring).  Per 64-key tile: S^T = K Q^T and dP^T = V dY^T of both
//    32-key halves (four independent MFMA chains), dS^T in registers,
//    dQ^T += K^T dS^T (K^T by the transposing read).  The linear branch is
//    added at the end from S_t (transposed layout, bf16 hi/lo) and z_t.
// fp32 kernels: the same sums on the vector ALU (one query or key per lane).
#include <type_traits>

#include "local_common.h"

namespace rehyat {

namespace {

#ifndef REHYAT_BWD_QWAVES
#define REHYAT_BWD_QWAVES 8
#endif
#ifndef REHYAT_BWD_QROWS
#define REHYAT_BWD_QROWS 64
#endif
constexpr int kBwdQWaves = REHYAT_BWD_QWAVES;  // waves of a dq workgroup (32 queries each)
constexpr int kBwdKeys = 128;                  // keys per dk/dv workgroup (4 pairs of waves)
constexpr int kBwdQRows = REHYAT_BWD_QROWS;    // query rows per dk/dv LDS tile
constexpr int kBwdQueries = 32 * kBwdQWaves;   // queries per dq workgroup
// keys per dq LDS tile, taken in 64-key halves between barriers: 128 for elu+1
// (half the barriers: the whole backward 0.7 % faster, same results); 64 for
// the other maps, whose instances would spill with the larger ring
constexpr int dq_key_tile(int phi) { return phi == kPhiElu1 ? 128 : 64; }

// elu(x) + 1 and its derivative
__device__ __forceinline__ float elu1_grad(float x) { return x > 0.0f ? 1.0f : __expf(x); }

// dsum_i = dy_i . out_i: D/4 or D/8 lanes per row (16 bytes of dy each),
// reduced by shuffles.  T: dy's type; U: out's (the bf16 path's fp32 copy of
// the output, when the caller kept it, else bf16).
template <int D, typename T, typename U>
__global__ __launch_bounds__(256) void dsum_kernel(const T* __restrict__ dy, const U* __restrict__ out,
                                                   float* __restrict__ dsum, long long rows) {
    constexpr int EPL = 16 / sizeof(T);  // elements per lane
    constexpr int LPR = D / EPL;         // lanes per row
    const long long g = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long row = g / LPR;
    const int part = (int)(g % LPR);
    float acc = 0.0f;
    if (row < rows) {
        float x[EPL], y[EPL];
        const u32x4 a = *(const u32x4*)(dy + row * D + part * EPL);
        if constexpr (sizeof(T) == 2) unpack8(a, x);
        else
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = __uint_as_float(a[e]);
#pragma unroll
        for (int o = 0; o < EPL * (int)sizeof(U) / 16; ++o) {
            const u32x4 b = *(const u32x4*)(out + row * D + part * EPL + o * (16 / sizeof(U)));
            if constexpr (sizeof(U) == 2) unpack8(b, y);
            else
#pragma unroll
                for (int e = 0; e < 4; ++e) y[4 * o + e] = __uint_as_float(b[e]);
        }
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc += x[e] * y[e];
    }
#pragma unroll
    for (int o = LPR / 2; o >= 1; o /= 2) acc += __shfl_xor(acc, o, LPR);
    if (row < rows && part == 0) dsum[row] = acc;
}

// Window [w0, w1) of the chunk of query row i (recurrent partition).
__device__ __forceinline__ void row_window(const BwdParams& p, int i, int& w0, int& w1) {
    const int t = i / (p.Tc * p.HW);
    w0 = max(t * p.Tc - p.To, 0) * p.HW;
    w1 = min((t + 1) * p.Tc, p.F) * p.HW;
}

// phi'(x) times the gradient of feature f (f < D: the elu+1 part, else the square part)
template <int D>
__device__ __forceinline__ float feature_grad(int f, float x, float g) {
    return f < D ? elu1_grad(x) * g : 2.0f * x * g;
}

// Load 4 consecutive bf16 and return them as floats.
__device__ __forceinline__ void load4_bf16(const uint16_t* p, float* f) {
    const u32x2 w = *(const u32x2*)p;
    f[0] = __uint_as_float(w[0] << 16);
    f[1] = __uint_as_float(w[0] & 0xffff0000u);
    f[2] = __uint_as_float(w[1] << 16);
    f[3] = __uint_as_float(w[1] & 0xffff0000u);
}

// ------------------------------------------------------------------ dk / dv (bf16)
// Each workgroup owns 128 keys and streams the query rows of the chunks whose
// windows hold them.  The work of a key is split over two waves: 4 pairs of
// waves, pair w owning keys kb0 + 32 w .. + 31 (one per lane).  The
// first wave of a pair forms S^T = K Q^T, P = exp(S - lse) on the key's
// windows and dV^T += dY^T P, and hands P (bf16, in the MFMA output layout) to
// the second wave through LDS; the second, one query tile behind, forms
// dP^T = V dY^T, dS = P (dP - dsum) and dK^T += Q^T dS.  Each wave holds one of
// K and V and one of the dV and dK accumulators, so two waves fit per SIMD and
// the vector work of one overlaps the products of the other.  Query tiles
// stream through a 3-stage LDS ring (the second wave reads the tile before).
template <int D, int PHI>
__global__ __launch_bounds__(512) void dkdv_bf16_kernel(BwdParams p) {
    constexpr int NP = 4, NW = 2 * NP, BQ = kBwdQRows, NST = 3, NQS = BQ / 32;
    static_assert(32 * NP == kBwdKeys, "a pair of waves per 32 keys of the block");
    constexpr int C = D / 8, KS = D / 16, DT = D / 32;
    constexpr int DP = PHI == kPhiElu1 ? D : 2 * D;
    constexpr int KSL = DP / 16, FT = DP / 32;
    constexpr int QT = BQ * D;                         // elements of a Q (or dY) tile
    constexpr int NI = QT * 2 / 1024;                  // 1 KB loads per tile
    constexpr int OPW = 2 * NI / NW;                   // per wave, Q and dY
    static_assert(2 * NI % NW == 0, "tile loads must split evenly");
    __shared__ __attribute__((aligned(16))) uint16_t tiles_raw[NST][2 * QT];
    __shared__ __attribute__((aligned(16))) u32x4 pbuf[2][NP][NQS][2][64];  // P of a tile, per pair
    __shared__ __attribute__((aligned(16))) float rowf[NST][2][BQ];        // lse log2(e), dsum
    __shared__ __attribute__((aligned(16))) int roww[NST][2][BQ];          // window bounds

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool first = wave < NP;                      // S, P, dV (else dP, dS, dK)
    const int pair = wave % NP;
    const int h = lane >> 5, lq = lane & 31;
    const int nkb = (p.N + kBwdKeys - 1) / kBwdKeys;
    const int item = __builtin_amdgcn_readfirstlane(xcd_remap(blockIdx.x, gridDim.x));
    const int bh = item / nkb;
    const int kb0 = (item - bh * nkb) * kBwdKeys;
    const int key = kb0 + 32 * pair + lq;              // the lane's key (column of every tile)
    const bool key_ok = key < p.N;
    const int keyc = min(key, p.N - 1);

    const uint16_t* qb = (const uint16_t*)p.q + bh * p.bh_stride;
    const uint16_t* kbp = (const uint16_t*)p.k + bh * p.bh_stride;
    const uint16_t* vbp = (const uint16_t*)p.v + bh * p.bh_stride;
    const uint16_t* dyb = (const uint16_t*)p.dy + bh * p.bh_stride;
    const float* lseb = p.lse + (long long)bh * p.N;
    const float* dsb = p.dsum + (long long)bh * p.N;

    // the first wave of a pair holds K of its keys, the second V
    bf16x8 kv[KS];
    {
        const uint16_t* src = (first ? kbp : vbp) + (long long)keyc * D + 8 * h;
#pragma unroll
        for (int s = 0; s < KS; ++s) kv[s] = __builtin_bit_cast(bf16x8, ldg_b128(src + 16 * s));
    }

    // query rows of the chunks whose windows hold any of the block's keys
    const int kl = min(kb0 + kBwdKeys, p.N) - 1;
    const int fa = kb0 / p.HW, fb = kl / p.HW;
    const int t_lo = fa / p.Tc, t_hi = min((fb + p.To) / p.Tc, p.C - 1);
    const int qr0 = t_lo * p.Tc * p.HW;
    const int qr1 = min((t_hi + 1) * p.Tc, p.F) * p.HW;
    const int ntiles = (qr1 - qr0 + BQ - 1) / BQ;

    const int rb = D * 2;
    const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc((void*)qb, (short)0, qr1 * rb, 0x00020000);
    const __amdgpu_buffer_rsrc_t dyrs = __builtin_amdgcn_make_buffer_rsrc((void*)dyb, (short)0, qr1 * rb, 0x00020000);
    auto load_tile = [&](int st, int it) {
        const int r0 = qr0 + it * BQ;
#pragma unroll
        for (int o = 0; o < OPW; ++o) {
            const int op = wave + o * NW;
            const bool isdy = op >= NI;
            const int ins = isdy ? op - NI : op;
            const int pos = 64 * ins + lane;
            const int r = pos / C;
            const int off = (r0 + r) * rb + ((pos % C) ^ swz<C>(r)) * 16;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(isdy ? dyrs : qrs,
                                                     (__attribute__((address_space(3))) void*)(
                                                         (lds_u16*)tiles_raw[st] + (isdy ? QT : 0) + 512 * ins),
                                                     16, off, 0, 0, 0);
        }
    };
    // per-row data of a tile: waves 0 .. BQ/64-1 load it into registers (one
    // row per lane) and store it after the current tile
    static_assert(BQ % 64 == 0 && BQ / 64 <= NW, "row data: one row per lane of the first waves");
    constexpr int RW = BQ / 64;
    float rl = 0.0f, rd = 0.0f;
    int rw0 = 0, rw1 = 0;
    auto fetch_rows = [&](int it) {
        const int i = qr0 + it * BQ + 64 * wave + lane;
        if (i < qr1) {
            rl = lseb[i] * kLog2e;
            rd = dsb[i];
            row_window(p, i, rw0, rw1);
        } else {
            rl = rd = 0.0f;
            rw0 = rw1 = 0;  // no key lies in an empty window
        }
    };
    auto store_rows = [&](int st) {
        rowf[st][0][64 * wave + lane] = rl;
        rowf[st][1][64 * wave + lane] = rd;
        roww[st][0][64 * wave + lane] = rw0;
        roww[st][1][64 * wave + lane] = rw1;
    };

    // transposing-read offsets (dY^T / Q^T fragments: lane row d = 32 c + lq,
    // query rows 4h..4h+3 and 8+4h..8+4h+3 of a 16-row step)
    const int tr_row = 4 * h + ((lane & 15) >> 2);
    const int tr_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    const int tr_sub = 4 * (lane & 1);
    int toff[DT][2];
#pragma unroll
    for (int c = 0; c < DT; ++c) {
        const int ch = 4 * c + tr_chunk;
        toff[c][0] = tr_row * D + ((ch ^ swz<C>(tr_row)) << 3) + tr_sub;
        toff[c][1] = (tr_row + 8) * D + ((ch ^ swz<C>(tr_row + 8)) << 3) + tr_sub;
    }

    f32x16 acc[DT];  // dV^T (first wave) or dK^T (second)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};

    // ---- linear branch of the keys (delta blocks u <= C-2, or the 2C+1
    // bidirectional blocks): dv += G_u^T phi(k) on the first wave, dk from
    // dphi(k) = G_u v - g_u on the second
    if constexpr (PHI != kPhiNone) {
        if (p.lin) {
            const bool bidir = p.mode == kBidirectional;
            const int u_key = bidir ? bidir_block_of_frame(keyc / p.HW, p.Tc, p.To) : (keyc / p.HW + p.To) / p.Tc;
            const int u_first = __builtin_amdgcn_readfirstlane(u_key);
            const int u_last = __shfl(u_key, 31);
            const int u_max = bidir ? 2 * p.C : p.C - 2;
            const int slots = bidir ? 2 * p.C + 1 : p.C;
            for (int u = u_first; u <= u_last && u <= u_max; ++u) {
                const bool mine = key_ok && u_key == u;
                const long long sofs = (long long)bh * slots * p.s_stride + (long long)u * p.s_stride;
                if (first) {
                    const uint16_t* ghi = (const uint16_t*)p.g_hi + sofs;
                    const uint16_t* glo = (const uint16_t*)p.g_lo + sofs;
#pragma unroll 1
                    for (int dt = 0; dt < DT; ++dt) {
                        f32x16 a = f32x16{};
#pragma unroll
                        for (int ksl = 0; ksl < KSL; ++ksl) {
                            // phi(k) is recomputed for every output tile: held
                            // for all of them it would not fit in the registers
                            u32x4 kx = __builtin_bit_cast(u32x4, kv[ksl % KS]);
                            asm volatile("" : "+v"(kx));
                            float x[8], f[8];
                            unpack8(kx, x);
#pragma unroll
                            for (int e = 0; e < 8; ++e) f[e] = mine ? (ksl < KS ? elu1(x[e]) : x[e] * x[e]) : 0.0f;
                            u32x4 whi, wlo;
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const u32x2 hl = split2_bf16(f[2 * e], f[2 * e + 1]);
                                whi[e] = hl[0];
                                wlo[e] = hl[1];
                            }
                            const long long off = (long long)(32 * dt + lq) * DP + 16 * ksl + 8 * h;
                            const bf16x8 ah = __builtin_bit_cast(bf16x8, ldg_b128(ghi + off));
                            const bf16x8 al = __builtin_bit_cast(bf16x8, ldg_b128(glo + off));
                            const bf16x8 fh = __builtin_bit_cast(bf16x8, whi), fl = __builtin_bit_cast(bf16x8, wlo);
                            a = mfma32x32x16(ah, fh, a);
                            a = mfma32x32x16(al, fh, a);
                            a = mfma32x32x16(ah, fl, a);
                        }
#pragma unroll
                        for (int x = 0; x < DT; ++x)  // static register indices (dt is not unrolled)
                            if (x == dt) acc[x] += a;
                    }
                } else {
                    const uint16_t* gthi = (const uint16_t*)p.gt_hi + sofs;
                    const uint16_t* gtlo = (const uint16_t*)p.gt_lo + sofs;
                    const float* gz = p.gz + (long long)bh * slots * p.z_stride + (long long)u * p.z_stride;
#pragma unroll 1
                    for (int ft = 0; ft < FT; ++ft) {
                        f32x16 a = f32x16{};
#pragma unroll
                        for (int s = 0; s < KS; ++s) {
                            const long long off = (long long)(32 * ft + lq) * D + 16 * s + 8 * h;
                            a = mfma32x32x16(__builtin_bit_cast(bf16x8, ldg_b128(gthi + off)), kv[s], a);
                            a = mfma32x32x16(__builtin_bit_cast(bf16x8, ldg_b128(gtlo + off)), kv[s], a);
                        }
                        if (!mine) continue;
                        const int dt = ft % DT;
                        f32x16 add;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int f0 = 32 * ft + 8 * j + 4 * h;          // features f0 .. f0+3
                            const int d0 = 32 * dt + 8 * j + 4 * h;          // their head_dim rows
                            const f32x4 g4 = *(const f32x4*)(gz + f0);
                            float kx[4];
                            load4_bf16(kbp + (long long)keyc * D + d0, kx);
#pragma unroll
                            for (int i = 0; i < 4; ++i) add[4 * j + i] = feature_grad<D>(f0 + i, kx[i], a[4 * j + i] - g4[i]);
                        }
#pragma unroll
                        for (int x = 0; x < DT; ++x)
                            if (x == dt) acc[x] += add;
                    }
                }
            }
        }
    }

    // first wave, tile t: S^T, P (masked to the windows), P to LDS, dV^T += dY^T P
    // (FULL: every key of the block lies in the window of every row of the tile,
    // no masking needed; one instance each, so that neither has a branch inside)
    auto first_step = [&](int t, auto full_c) {
        constexpr bool FULL = decltype(full_c)::value;
        // the first role's loop keeps its read addresses live across the loop
        // (its own loop has the registers for them; the second role's does not)
        int ln = lane;
        const int h = ln >> 5, lq = ln & 31;
        int toff[DT][2];
        {
            const int tr_row = 4 * h + ((ln & 15) >> 2);
            const int tr_chunk = 2 * ((ln >> 4) & 1) + ((ln & 3) >> 1);
            const int tr_sub = 4 * (ln & 1);
#pragma unroll
            for (int c = 0; c < DT; ++c) {
                const int ch = 4 * c + tr_chunk;
                toff[c][0] = tr_row * D + ((ch ^ swz<C>(tr_row)) << 3) + tr_sub;
                toff[c][1] = (tr_row + 8) * D + ((ch ^ swz<C>(tr_row + 8)) << 3) + tr_sub;
            }
        }
        const int st = t % NST;
        const lds_u16* Qs = (const lds_u16*)tiles_raw[st];
        const lds_u16* Ys = Qs + QT;
        asm volatile("" : "+v"(Ys));  // the two tiles' reads keep bases of their own
        // the subtiles' S^T chains side by side (independent accumulators)
        f32x16 sall[NQS];
#pragma unroll
        for (int qs = 0; qs < NQS; ++qs) sall[qs] = f32x16{};
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int qs = 0; qs < NQS; ++qs) {
                const int arow = 32 * qs + lq;
                const int off = arow * D + (((2 * s + h) ^ swz<C>(arow)) << 3);
                sall[qs] = mfma32x32x16(lds_read_b128(Qs, off), kv[s], sall[qs]);
            }
#pragma unroll
        for (int qs = 0; qs < NQS; ++qs) {
            const f32x16& sacc = sall[qs];
            // rows 32 qs + 8 j + 4 h + i of the tile, column = the lane's key
            u32x4 pw[2];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r0 = 32 * qs + 8 * j + 4 * h;
                const f32x4 l4 = *(const __attribute__((address_space(3))) f32x4*)&rowf[st][0][r0];
                float pv[4];
                if constexpr (FULL) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) pv[i] = __builtin_amdgcn_exp2f(sacc[4 * j + i] * kLog2e - l4[i]);
                } else {
                    typedef int i32x4 __attribute__((ext_vector_type(4)));
                    const i32x4 a4 = *(const __attribute__((address_space(3))) i32x4*)&roww[st][0][r0];
                    const i32x4 b4 = *(const __attribute__((address_space(3))) i32x4*)&roww[st][1][r0];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const bool in = key_ok && key >= a4[i] && key < b4[i];
                        pv[i] = in ? __builtin_amdgcn_exp2f(sacc[4 * j + i] * kLog2e - l4[i]) : 0.0f;
                    }
                }
                pw[j >> 1][2 * (j & 1)] = pack2_bf16(pv[0], pv[1]);
                pw[j >> 1][2 * (j & 1) + 1] = pack2_bf16(pv[2], pv[3]);
            }
            pbuf[t & 1][pair][qs][0][ln] = pw[0];
            pbuf[t & 1][pair][qs][1][ln] = pw[1];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int r16 = (32 * qs + 16 * kk) * D;
                const bf16x8 pb = __builtin_bit_cast(bf16x8, pw[kk]);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const bf16x8 ya = cat(lds_read_tr(Ys, r16 + toff[dt][0]), lds_read_tr(Ys, r16 + toff[dt][1]));
                    acc[dt] = mfma32x32x16(ya, pb, acc[dt]);
                }
            }
        }
    };
    // second wave, tile t: dP^T, dS = P (dP - dsum) with the first wave's P, dK^T += Q^T dS
    auto second_step = [&](int t) {
        // lane addressing re-derived per step behind an empty asm, so that the
        // compiler does not keep every read's address live across the loop
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int h = ln >> 5, lq = ln & 31;
        int toff[DT][2];
        {
            const int tr_row = 4 * h + ((ln & 15) >> 2);
            const int tr_chunk = 2 * ((ln >> 4) & 1) + ((ln & 3) >> 1);
            const int tr_sub = 4 * (ln & 1);
#pragma unroll
            for (int c = 0; c < DT; ++c) {
                const int ch = 4 * c + tr_chunk;
                toff[c][0] = tr_row * D + ((ch ^ swz<C>(tr_row)) << 3) + tr_sub;
                toff[c][1] = (tr_row + 8) * D + ((ch ^ swz<C>(tr_row + 8)) << 3) + tr_sub;
            }
        }
        const int st = t % NST;
        const lds_u16* Qs = (const lds_u16*)tiles_raw[st];
        const lds_u16* Ys = Qs + QT;
        asm volatile("" : "+v"(Ys));  // the two tiles' reads keep bases of their own
        f32x16 pall[NQS];
#pragma unroll
        for (int qs = 0; qs < NQS; ++qs) pall[qs] = f32x16{};
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int qs = 0; qs < NQS; ++qs) {
                const int arow = 32 * qs + lq;
                const int off = arow * D + (((2 * s + h) ^ swz<C>(arow)) << 3);
                pall[qs] = mfma32x32x16(lds_read_b128(Ys, off), kv[s], pall[qs]);
            }
#pragma unroll
        for (int qs = 0; qs < NQS; ++qs) {
            const f32x16& pacc = pall[qs];
            const u32x4 pw[2] = {pbuf[t & 1][pair][qs][0][ln], pbuf[t & 1][pair][qs][1][ln]};
            u32x4 dw[2];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r0 = 32 * qs + 8 * j + 4 * h;
                const f32x4 d4 = *(const __attribute__((address_space(3))) f32x4*)&rowf[st][1][r0];
                const uint32_t w0 = pw[j >> 1][2 * (j & 1)], w1 = pw[j >> 1][2 * (j & 1) + 1];
                const float pv[4] = {__uint_as_float(w0 << 16), __uint_as_float(w0 & 0xffff0000u),
                                     __uint_as_float(w1 << 16), __uint_as_float(w1 & 0xffff0000u)};
                float dv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) dv[i] = pv[i] * (pacc[4 * j + i] - d4[i]);
                dw[j >> 1][2 * (j & 1)] = pack2_bf16(dv[0], dv[1]);
                dw[j >> 1][2 * (j & 1) + 1] = pack2_bf16(dv[2], dv[3]);
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int r16 = (32 * qs + 16 * kk) * D;
                const bf16x8 db = __builtin_bit_cast(bf16x8, dw[kk]);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const bf16x8 qa = cat(lds_read_tr(Qs, r16 + toff[dt][0]), lds_read_tr(Qs, r16 + toff[dt][1]));
                    acc[dt] = mfma32x32x16(qa, db, acc[dt]);
                }
            }
        }
    };

    if (ntiles > 0) {
        load_tile(0, 0);
        if (wave < RW) {
            fetch_rows(0);
            store_rows(0);
        }
    }
    // iteration it: the first waves take tile it, the second waves tile it - 1;
    // the ring holds tiles it - 1, it and (being loaded) it + 1.  Each role has
    // a loop of its own (the same barriers, one per iteration): in one loop
    // shared by both, the accumulators of the two roles' paths were given
    // different registers and copied over (32 64-bit moves) every iteration.
    auto iteration_start = [&](int it) {
        // own loads of tile it and own LDS writes (P, row data) have landed,
        // then every wave's have
        __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
        lds_barrier();
        const bool more = it + 1 < ntiles;
        if (more) {
            load_tile((it + 1) % NST, it + 1);
            if (wave < RW) fetch_rows(it + 1);
        }
        return more;
    };
    if (first) {
        for (int it = 0; it <= ntiles && ntiles > 0; ++it) {
            const bool more = iteration_start(it);
            if (it < ntiles) {
                // windows move forward with the row: the tile needs no mask when
                // its first row's window ends after the block and its last row's
                // starts before it
                const int ia = qr0 + it * BQ, ib = ia + BQ - 1;
                int a0, a1, b0, b1;
                row_window(p, ia, a0, a1);
                row_window(p, ib, b0, b1);
                if (ib < qr1 && kb0 + kBwdKeys <= p.N && b0 <= kb0 && a1 >= kb0 + kBwdKeys)
                    first_step(it, std::true_type{});
                else
                    first_step(it, std::false_type{});
            }
            if (more && wave < RW) store_rows((it + 1) % NST);
        }
    } else {
        for (int it = 0; it <= ntiles && ntiles > 0; ++it) {
            const bool more = iteration_start(it);
            if (it > 0) second_step(it - 1);
            if (more && wave < RW) store_rows((it + 1) % NST);
        }
    }

    if (!key_ok) return;
    uint16_t* dst = (uint16_t*)(first ? p.dv : p.dk) + bh * p.bh_stride + (long long)key * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int d0 = 32 * dt + 8 * j + 4 * h;
            *(u32x2*)(dst + d0) = u32x2{pack2_bf16(acc[dt][4 * j], acc[dt][4 * j + 1]),
                                        pack2_bf16(acc[dt][4 * j + 2], acc[dt][4 * j + 3])};
        }
}

// ------------------------------------------------------------------ dq (bf16)
template <int D, int PHI>
__global__ __launch_bounds__(kBwdQWaves * 64) void dq_bf16_kernel(BwdParams p, int tiles_per_chunk) {
    constexpr int NW = kBwdQWaves, BN = dq_key_tile(PHI);
    constexpr int C = D / 8, KS = D / 16, DT = D / 32;
    constexpr int DP = PHI == kPhiElu1 ? D : 2 * D;
    constexpr int FT = DP / 32;
    constexpr int KT = BN * D;                          // elements of a K (or V) tile
    constexpr int NI = KT * 2 / 1024;
    constexpr int OPW = 2 * NI / NW;
    static_assert(2 * NI % NW == 0, "tile loads must split evenly");
    __shared__ __attribute__((aligned(16))) uint16_t tiles_raw[2][2 * KT];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, lq = lane & 31;
    // items (b, h, chunk, query tile) in the local kernel's order: each XCD owns
    // a contiguous share, optionally taken longest window first
    LocalParams wl{};
    wl.F = p.F; wl.Tc = p.Tc; wl.To = p.To; wl.HW = p.HW;
    wl.n_chunks = p.C; wl.tiles_per_chunk = tiles_per_chunk; wl.lpt_order = p.dq_lpt;
    const int item = __builtin_amdgcn_readfirstlane(local_work_item(wl, blockIdx.x, gridDim.x, BN));
    const int per_bh = p.C * tiles_per_chunk;
    const int bh = item / per_bh;
    const int rem = item - bh * per_bh;
    const int t = rem / tiles_per_chunk;
    const int tile = rem - t * tiles_per_chunk;
    const int q_end = min((t + 1) * p.Tc, p.F) * p.HW;
    const int q0 = t * p.Tc * p.HW + tile * kBwdQueries;
    if (q0 >= q_end) return;
    const int w0 = max(t * p.Tc - p.To, 0) * p.HW;
    const int nkeys = q_end - w0;
    const int ntiles = (nkeys + BN - 1) / BN;
    const int row = q0 + 32 * wave + lq;                 // the lane's query
    const bool row_ok = row < q_end;
    const int rowc = min(row, q_end - 1);

    const uint16_t* qb = (const uint16_t*)p.q + bh * p.bh_stride;
    const uint16_t* dyb = (const uint16_t*)p.dy + bh * p.bh_stride;
    const uint16_t* kbp = (const uint16_t*)p.k + bh * p.bh_stride + (long long)w0 * D;
    const uint16_t* vbp = (const uint16_t*)p.v + bh * p.bh_stride + (long long)w0 * D;
    const float lse = p.lse[(long long)bh * p.N + rowc];
    const float dsum = p.dsum[(long long)bh * p.N + rowc];
    const float lse2 = lse * kLog2e;

    bf16x8 qf[KS], yf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        qf[s] = __builtin_bit_cast(bf16x8, ldg_b128(qb + (long long)rowc * D + 16 * s + 8 * h));
        yf[s] = __builtin_bit_cast(bf16x8, ldg_b128(dyb + (long long)rowc * D + 16 * s + 8 * h));
    }

    const int rb = D * 2;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)kbp, (short)0, nkeys * rb, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vbp, (short)0, nkeys * rb, 0x00020000);
    auto load_tile = [&](lds_u16* dst, int it) {
#pragma unroll
        for (int o = 0; o < OPW; ++o) {
            const int op = wave + o * NW;
            const bool isv = op >= NI;
            const int ins = isv ? op - NI : op;
            const int pos = 64 * ins + lane;
            const int r = pos / C;
            const int off = (it * BN + r) * rb + ((pos % C) ^ swz<C>(r)) * 16;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(isv ? vrs : krs,
                                                     (__attribute__((address_space(3))) void*)(dst + (isv ? KT : 0) + 512 * ins),
                                                     16, off, 0, 0, 0);
        }
    };
    const int tr_row = 4 * h + ((lane & 15) >> 2);
    const int tr_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    const int tr_sub = 4 * (lane & 1);
    int toff[DT][2];
#pragma unroll
    for (int c = 0; c < DT; ++c) {
        const int ch = 4 * c + tr_chunk;
        toff[c][0] = tr_row * D + ((ch ^ swz<C>(tr_row)) << 3) + tr_sub;
        toff[c][1] = (tr_row + 8) * D + ((ch ^ swz<C>(tr_row + 8)) << 3) + tr_sub;
    }

    f32x16 dqt[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) dqt[dt] = f32x16{};

    // one key tile; TAIL: the window's last tile, the only one whose keys can
    // run past the window end (the others carry no key test)
    auto tile_step = [&](auto tail, int it) {
        constexpr bool TAIL = decltype(tail)::value;
        const int buf = it & 1;
        __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
        lds_barrier();
        // the slot being filled and the slot being read never overlap; as
        // restrict pointers they keep the reads clear of a wait for the loads
        auto body = [&](lds_u16* __restrict__ fill, const lds_u16* __restrict__ Ks) {
        if (it + 1 < ntiles) load_tile(fill, it + 1);
        const lds_u16* Vs0 = Ks + KT;
        for (int hf = 0; hf < BN / 64; ++hf) {
        const lds_u16* Kh = Ks + 64 * hf * D;
        const lds_u16* Vs = Vs0 + 64 * hf * D;
        // the S^T and dP^T chains of every 32-key subtile side by side
        constexpr int NKS = 2;
        f32x16 sall[NKS], pall[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) sall[ks] = pall[ks] = f32x16{};
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const int arow = 32 * ks + lq;
                const int off = arow * D + (((2 * s + h) ^ swz<C>(arow)) << 3);
                sall[ks] = mfma32x32x16(lds_read_b128(Kh, off), qf[s], sall[ks]);
                pall[ks] = mfma32x32x16(lds_read_b128(Vs, off), yf[s], pall[ks]);
            }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const f32x16& sacc = sall[ks];
            const f32x16& pacc = pall[ks];
            // key rows 32 ks + 8 j + 4 h + i of the tile, column = the lane's query
            u32x4 dw[2];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float dv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int kr = it * BN + 64 * hf + 32 * ks + 8 * j + 4 * h + i;
                    const float pe = !TAIL || kr < nkeys ? __builtin_amdgcn_exp2f(sacc[4 * j + i] * kLog2e - lse2) : 0.0f;
                    dv[i] = pe * (pacc[4 * j + i] - dsum);
                }
                dw[j >> 1][2 * (j & 1)] = pack2_bf16(dv[0], dv[1]);
                dw[j >> 1][2 * (j & 1) + 1] = pack2_bf16(dv[2], dv[3]);
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int r16 = (32 * ks + 16 * kk) * D;
                const bf16x8 db = __builtin_bit_cast(bf16x8, dw[kk]);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const bf16x8 ka = cat(lds_read_tr(Kh, r16 + toff[dt][0]), lds_read_tr(Kh, r16 + toff[dt][1]));
                    dqt[dt] = mfma32x32x16(ka, db, dqt[dt]);
                }
            }
        }
        }
        };
        body((lds_u16*)tiles_raw[buf ^ 1], (const lds_u16*)tiles_raw[buf]);
    };
    if (ntiles > 0) load_tile((lds_u16*)tiles_raw[0], 0);
    for (int it = 0; it < ntiles - 1; ++it) tile_step(std::false_type{}, it);
    if (ntiles > 0) tile_step(std::true_type{}, ntiles - 1);

    // ---- linear branch: dphi(q) = e^{-lse} (S_t dy - D z_t)
    if constexpr (PHI != kPhiNone) {
        if (p.lin && (p.mode == kBidirectional || t * p.Tc - p.To > 0)) {
            const long long sofs = (long long)bh * p.C * p.s_stride + (long long)t * p.s_stride;
            const uint16_t* sthi = (const uint16_t*)p.st_hi + sofs;
            const uint16_t* stlo = (const uint16_t*)p.st_lo + sofs;
            const float* zt = p.z + (long long)bh * p.C * p.z_stride + (long long)t * p.z_stride;
            const float el = __expf(-lse);
#pragma unroll
            for (int ft = 0; ft < FT; ++ft) {
                f32x16 acc = f32x16{};
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    const long long off = (long long)(32 * ft + lq) * D + 16 * s + 8 * h;
                    acc = mfma32x32x16(__builtin_bit_cast(bf16x8, ldg_b128(sthi + off)), yf[s], acc);
                    acc = mfma32x32x16(__builtin_bit_cast(bf16x8, ldg_b128(stlo + off)), yf[s], acc);
                }
                const int dt = ft % DT;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int f0 = 32 * ft + 8 * j + 4 * h;
                    const int d0 = 32 * dt + 8 * j + 4 * h;
                    const f32x4 z4 = *(const f32x4*)(zt + f0);
                    float qx[4];
                    load4_bf16(qb + (long long)rowc * D + d0, qx);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        dqt[dt][4 * j + i] += feature_grad<D>(f0 + i, qx[i], el * (acc[4 * j + i] - dsum * z4[i]));
                }
            }
        }
    }

    if (!row_ok) return;
    uint16_t* dqp = (uint16_t*)p.dq + bh * p.bh_stride + (long long)row * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int d0 = 32 * dt + 8 * j + 4 * h;
            *(u32x2*)(dqp + d0) = u32x2{pack2_bf16(dqt[dt][4 * j], dqt[dt][4 * j + 1]),
                                        pack2_bf16(dqt[dt][4 * j + 2], dqt[dt][4 * j + 3])};
        }
}

// ------------------------------------------------------------------ fp32
constexpr int kF32Lanes = 64;

// dk, dv: one key per lane; query rows of the chunks whose windows hold the
// workgroup's keys stream through LDS 32 at a time.
template <int D, int PHI>
__global__ __launch_bounds__(kF32Lanes) void dkdv_f32_kernel(BwdParams p) {
    constexpr int R = 32;
    constexpr int DP = PHI == kPhiElu1 ? D : 2 * D;
    __shared__ float Qs[R][D], Ys[R][D];
    __shared__ float Ls[R], Ds[R];
    __shared__ int W0[R], W1[R];
    const int nkb = (p.N + kF32Lanes - 1) / kF32Lanes;
    const int bh = blockIdx.x / nkb;
    const int kb0 = (blockIdx.x - bh * nkb) * kF32Lanes;
    const int tid = threadIdx.x;
    const int key = kb0 + tid;
    const bool key_ok = key < p.N;
    const int keyc = min(key, p.N - 1);
    const float* qb = (const float*)p.q + bh * p.bh_stride;
    const float* kb = (const float*)p.k + bh * p.bh_stride;
    const float* vb = (const float*)p.v + bh * p.bh_stride;
    const float* yb = (const float*)p.dy + bh * p.bh_stride;
    float k[D], v[D], dk[D], dv[D];
#pragma unroll
    for (int c = 0; c < D; ++c) {
        k[c] = kb[(long long)keyc * D + c];
        v[c] = vb[(long long)keyc * D + c];
        dk[c] = 0.0f;
        dv[c] = 0.0f;
    }
    const int kl = min(kb0 + kF32Lanes, p.N) - 1;
    const int t_lo = (kb0 / p.HW) / p.Tc, t_hi = min((kl / p.HW + p.To) / p.Tc, p.C - 1);
    const int qr0 = t_lo * p.Tc * p.HW, qr1 = min((t_hi + 1) * p.Tc, p.F) * p.HW;
    for (int r0 = qr0; r0 < qr1; r0 += R) {
        __syncthreads();
        for (int e = tid; e < R * D; e += kF32Lanes) {
            const int r = e / D, c = e % D;
            const int i = r0 + r;
            Qs[r][c] = i < qr1 ? qb[(long long)i * D + c] : 0.0f;
            Ys[r][c] = i < qr1 ? yb[(long long)i * D + c] : 0.0f;
        }
        if (tid < R) {
            const int i = r0 + tid;
            int a = 0, b = 0;
            if (i < qr1) row_window(p, i, a, b);
            Ls[tid] = i < qr1 ? p.lse[(long long)bh * p.N + i] : 0.0f;
            Ds[tid] = i < qr1 ? p.dsum[(long long)bh * p.N + i] : 0.0f;
            W0[tid] = a;
            W1[tid] = b;
        }
        __syncthreads();
        for (int r = 0; r < R; ++r) {
            if (!(key_ok && key >= W0[r] && key < W1[r])) continue;
            float s = 0.0f, dp = 0.0f;
#pragma unroll
            for (int c = 0; c < D; ++c) {
                s = fmaf(Qs[r][c], k[c], s);
                dp = fmaf(Ys[r][c], v[c], dp);
            }
            const float pe = expf(s - Ls[r]);
            const float ds = pe * (dp - Ds[r]);
#pragma unroll
            for (int c = 0; c < D; ++c) {
                dv[c] = fmaf(pe, Ys[r][c], dv[c]);
                dk[c] = fmaf(ds, Qs[r][c], dk[c]);
            }
        }
    }
    if (!key_ok) return;
    if (PHI != kPhiNone && p.lin) {
        const bool bidir = p.mode == kBidirectional;
        const int u = bidir ? bidir_block_of_frame(key / p.HW, p.Tc, p.To) : (key / p.HW + p.To) / p.Tc;
        const int slots = bidir ? 2 * p.C + 1 : p.C;
        if (bidir || u <= p.C - 2) {
            const long long sofs = (long long)bh * slots * p.s_stride + (long long)u * p.s_stride;
            const float* G = (const float*)p.gt_hi + sofs;   // [D'][d]
            const float* gz = p.gz + (long long)bh * slots * p.z_stride + (long long)u * p.z_stride;
            for (int f = 0; f < DP; ++f) {
                const float x = k[f % D];
                const float phi = f < D ? elu1(x) : x * x;
                float g = -gz[f];
#pragma unroll
                for (int c = 0; c < D; ++c) {
                    g = fmaf(G[(long long)f * D + c], v[c], g);
                    dv[c] = fmaf(G[(long long)f * D + c], phi, dv[c]);
                }
                dk[f % D] += feature_grad<D>(f, x, g);
            }
        }
    }
    float* dkp = (float*)p.dk + bh * p.bh_stride + (long long)key * D;
    float* dvp = (float*)p.dv + bh * p.bh_stride + (long long)key * D;
#pragma unroll
    for (int c = 0; c < D; ++c) {
        dkp[c] = dk[c];
        dvp[c] = dv[c];
    }
}

// dq: one query per lane; the window's keys stream through LDS 32 at a time.
template <int D, int PHI>
__global__ __launch_bounds__(kF32Lanes) void dq_f32_kernel(BwdParams p, int tiles_per_chunk) {
    constexpr int R = 32;
    constexpr int DP = PHI == kPhiElu1 ? D : 2 * D;
    __shared__ float Ks[R][D], Vs[R][D];
    const int per_bh = p.C * tiles_per_chunk;
    const int bh = blockIdx.x / per_bh;
    const int rem = blockIdx.x - bh * per_bh;
    const int t = rem / tiles_per_chunk;
    const int tile = rem - t * tiles_per_chunk;
    const int q_end = min((t + 1) * p.Tc, p.F) * p.HW;
    const int q0 = t * p.Tc * p.HW + tile * kF32Lanes;
    if (q0 >= q_end) return;
    const int tid = threadIdx.x;
    const int row = q0 + tid;
    const bool row_ok = row < q_end;
    const int rowc = min(row, q_end - 1);
    const int w0 = max(t * p.Tc - p.To, 0) * p.HW;
    const float* qb = (const float*)p.q + bh * p.bh_stride;
    const float* kb = (const float*)p.k + bh * p.bh_stride;
    const float* vb = (const float*)p.v + bh * p.bh_stride;
    const float* yb = (const float*)p.dy + bh * p.bh_stride;
    float q[D], y[D], dq[D];
#pragma unroll
    for (int c = 0; c < D; ++c) {
        q[c] = qb[(long long)rowc * D + c];
        y[c] = yb[(long long)rowc * D + c];
        dq[c] = 0.0f;
    }
    const float lse = p.lse[(long long)bh * p.N + rowc];
    const float dsum = p.dsum[(long long)bh * p.N + rowc];
    for (int j0 = w0; j0 < q_end; j0 += R) {
        __syncthreads();
        for (int e = tid; e < R * D; e += kF32Lanes) {
            const int r = e / D, c = e % D;
            const int j = j0 + r;
            Ks[r][c] = j < q_end ? kb[(long long)j * D + c] : 0.0f;
            Vs[r][c] = j < q_end ? vb[(long long)j * D + c] : 0.0f;
        }
        __syncthreads();
        for (int r = 0; r < R && j0 + r < q_end; ++r) {
            float s = 0.0f, dp = 0.0f;
#pragma unroll
            for (int c = 0; c < D; ++c) {
                s = fmaf(q[c], Ks[r][c], s);
                dp = fmaf(y[c], Vs[r][c], dp);
            }
            const float ds = expf(s - lse) * (dp - dsum);
#pragma unroll
            for (int c = 0; c < D; ++c) dq[c] = fmaf(ds, Ks[r][c], dq[c]);
        }
    }
    if (!row_ok) return;
    if (PHI != kPhiNone && p.lin && (p.mode == kBidirectional || t * p.Tc - p.To > 0)) {
        const long long sofs = (long long)bh * p.C * p.s_stride + (long long)t * p.s_stride;
        const float* S = (const float*)p.st_hi + sofs;   // [D'][d]
        const float* zt = p.z + (long long)bh * p.C * p.z_stride + (long long)t * p.z_stride;
        const float el = expf(-lse);
        for (int f = 0; f < DP; ++f) {
            float g = -dsum * zt[f];
#pragma unroll
            for (int c = 0; c < D; ++c) g = fmaf(S[(long long)f * D + c], y[c], g);
            dq[f % D] += feature_grad<D>(f, q[f % D], el * g);
        }
    }
    float* dqp = (float*)p.dq + bh * p.bh_stride + (long long)row * D;
#pragma unroll
    for (int c = 0; c < D; ++c) dqp[c] = dq[c];
}

int dq_tiles_per_chunk(const BwdParams& p, int rows) {
    const long long chunk_rows = (long long)min(p.Tc, p.F) * p.HW;
    return (int)((chunk_rows + rows - 1) / rows);
}

template <int D, int PHI>
hipError_t launch_bf16_dp(const BwdParams& p, hipStream_t s) {
    const long long kblocks = (long long)p.BH * ((p.N + kBwdKeys - 1) / kBwdKeys);
    const int tpc = dq_tiles_per_chunk(p, kBwdQueries);
    const long long qblocks = (long long)p.BH * p.C * tpc;
    if (kblocks > 0) dkdv_bf16_kernel<D, PHI><<<(unsigned)kblocks, 512, 0, s>>>(p);
    if (qblocks > 0) dq_bf16_kernel<D, PHI><<<(unsigned)qblocks, kBwdQWaves * 64, 0, s>>>(p, tpc);
    return hipGetLastError();
}

template <int D>
hipError_t launch_bf16_d(const BwdParams& p, hipStream_t s) {
    switch (p.phi) {
    case kPhiNone: return launch_bf16_dp<D, kPhiNone>(p, s);
    case kPhiElu1: return launch_bf16_dp<D, kPhiElu1>(p, s);
    case kPhiPoly2: return launch_bf16_dp<D, kPhiPoly2>(p, s);
    default: return hipErrorInvalidValue;
    }
}

template <int D, int PHI>
hipError_t launch_f32_dp(const BwdParams& p, hipStream_t s) {
    const long long kblocks = (long long)p.BH * ((p.N + kF32Lanes - 1) / kF32Lanes);
    const int tpc = dq_tiles_per_chunk(p, kF32Lanes);
    const long long qblocks = (long long)p.BH * p.C * tpc;
    if (kblocks > 0) dkdv_f32_kernel<D, PHI><<<(unsigned)kblocks, kF32Lanes, 0, s>>>(p);
    if (qblocks > 0) dq_f32_kernel<D, PHI><<<(unsigned)qblocks, kF32Lanes, 0, s>>>(p, tpc);
    return hipGetLastError();
}

template <int D>
hipError_t launch_f32_d(const BwdParams& p, hipStream_t s) {
    switch (p.phi) {
    case kPhiNone: return launch_f32_dp<D, kPhiNone>(p, s);
    case kPhiElu1: return launch_f32_dp<D, kPhiElu1>(p, s);
    case kPhiPoly2: return launch_f32_dp<D, kPhiPoly2>(p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

template <typename T, typename U>
static hipError_t dsum_typed(const BwdParams& p, const U* out, float* dsum, hipStream_t s) {
    const long long rows = (long long)p.BH * p.N;
    const int epl = 16 / (int)sizeof(T);
    const long long threads = rows * (p.d / epl);
    const unsigned blocks = (unsigned)((threads + 255) / 256);
    switch (p.d) {
    case 16: dsum_kernel<16, T, U><<<blocks, 256, 0, s>>>((const T*)p.dy, out, dsum, rows); break;
    case 32: dsum_kernel<32, T, U><<<blocks, 256, 0, s>>>((const T*)p.dy, out, dsum, rows); break;
    case 64: dsum_kernel<64, T, U><<<blocks, 256, 0, s>>>((const T*)p.dy, out, dsum, rows); break;
    case 128: dsum_kernel<128, T, U><<<blocks, 256, 0, s>>>((const T*)p.dy, out, dsum, rows); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_bwd_dsum(const BwdParams& p, float* dsum, bool bf16, hipStream_t s) {
    if (!bf16) return dsum_typed<float, float>(p, (const float*)p.out, dsum, s);
    if (p.out_f32) return dsum_typed<uint16_t, float>(p, p.out_f32, dsum, s);
    return dsum_typed<uint16_t, uint16_t>(p, (const uint16_t*)p.out, dsum, s);
}

void dq_launch_shape(const BwdParams& p, int& tiles_per_chunk, int& key_tile) {
    tiles_per_chunk = dq_tiles_per_chunk(p, kBwdQueries);
    key_tile = dq_key_tile(p.phi);
}

hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t s) {
    switch (p.d) {
    case 32: return launch_bf16_d<32>(p, s);
    case 64: return launch_bf16_d<64>(p, s);
    case 128: return launch_bf16_d<128>(p, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_bwd_f32(const BwdParams& p, hipStream_t s) {
    switch (p.d) {
    case 16: return launch_f32_d<16>(p, s);
    case 32: return launch_f32_d<32>(p, s);
    case 64: return launch_f32_d<64>(p, s);
    case 128: return launch_f32_d<128>(p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace rehyat
