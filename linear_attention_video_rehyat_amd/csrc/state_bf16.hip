// state_bf16.hip -- phi-map + block-state kernel (bf16 inputs, fp32 state).
//
// For each delta block E_u of keys (the keys that leave the softmax window
// between chunk u and chunk u+1) and each contiguous sub-block of it, computes
//   S^T_partial = sum_j v_j phi(k_j)^T   ([head_dim][D'], fp32)
//   z_partial   = sum_j phi(k_j)         ([D'], fp32)
// -- the cached linear-attention sums of ReHyAt §3.1 (arXiv 2601.04342),
// restricted to one block.  The cross-chunk scan adds them up into the state of
// each chunk (the §3.3 linear set is the union of the earlier delta blocks).
//
// phi is applied in fp32 and split into bf16 hi + lo parts so that the bf16
// MFMA products carry ~16 significant bits of phi(k); v is exact in bf16.
// z is summed on the vector ALU from the unsplit fp32 phi values.
// Both MFMA operands are read from row-major LDS tiles through the transposing
// LDS read (key index = contraction index).
#include "common.h"
#include "kernels.h"

namespace rehyat {

namespace {

template <int D, int PHI>
__global__ __launch_bounds__(256) void state_bf16_kernel(StateParams p) {
    constexpr int NW = 4;
    constexpr int DP = PHI == kPhiPoly2 ? 2 * D : D;
    constexpr int BN = 32;                        // keys per LDS tile
    constexpr int VP = tr_pitch(D);               // pitches (elements) for transposing reads
    constexpr int FP = tr_pitch(DP);
    constexpr int VT = BN * VP, FT = BN * FP;
    constexpr int BUF = VT + 2 * FT;              // one buffer: V, phi_hi, phi_lo
    constexpr int DT = D / 32, NT = DP / 32;
    constexpr int TILES = DT * NT;
    constexpr int TPW = (TILES + NW - 1) / NW;    // output tiles per wave
    constexpr int CHUNKS = BN * D / 8;            // 16-byte chunks per K or V tile
    constexpr int CPT = (CHUNKS + NW * 64 - 1) / (NW * 64);
    constexpr int E = D * DP + DP;

    __shared__ __attribute__((aligned(16))) uint16_t smem_raw[2 * BUF];
    __shared__ float zred[NW * 64][8];
    lds_u16* smem = (lds_u16*)smem_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h = lane >> 5;
    const int lq = lane & 31;

    // block -> (bh, u, sub)
    const int blk = blockIdx.x;
    const int per_bh = p.n_blocks * p.n_sub;
    const int bh = blk / per_bh;
    const int rem = blk - bh * per_bh;
    const int u = rem / p.n_sub;
    const int sub = rem - u * p.n_sub;

    int e0, e1;  // virtual key rows of the delta block
    if (p.stream_rows > 0) {
        e0 = 0;
        e1 = p.stream_rows;
    } else {
        e0 = max(u * p.Tc - p.To, 0) * p.HW;
        e1 = max((u + 1) * p.Tc - p.To, 0) * p.HW;
    }
    const int j0 = e0 + sub * p.sub_rows;
    const int j1 = min(j0 + p.sub_rows, e1);
    float* outp = p.partial + ((long long)(bh * p.n_blocks + u) * p.n_sub + sub) * E;

    const uint16_t* kb = (const uint16_t*)p.k + bh * p.bh_stride;
    const uint16_t* vb = (const uint16_t*)p.v + bh * p.bh_stride;
    const uint16_t* kpb = p.kp ? (const uint16_t*)p.kp + bh * p.prev_bh_stride : nullptr;
    const uint16_t* vpb = p.vp ? (const uint16_t*)p.vp + bh * p.prev_bh_stride : nullptr;

    f32x16 acc[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) acc[i] = f32x16{};
    float zacc[CPT][PHI == kPhiPoly2 ? 16 : 8];
#pragma unroll
    for (int i = 0; i < CPT; ++i)
#pragma unroll
        for (int c = 0; c < (PHI == kPhiPoly2 ? 16 : 8); ++c) zacc[i][c] = 0.0f;

    const int nrows = max(j1 - j0, 0);
    const int ntiles = (nrows + BN - 1) / BN;

    u32x4 kst[CPT], vst[CPT];
    auto load_tile = [&](int it) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tid + i * NW * 64;
            if (CHUNKS % (NW * 64) == 0 || c < CHUNKS) {
                const int r = c / (D / 8);
                const int col = (c % (D / 8)) * 8;
                const int j = min(j0 + it * BN + r, j1 - 1);
                if (j < p.prev_rows) {
                    kst[i] = ldg_b128(kpb + (long long)j * D + col);
                    vst[i] = ldg_b128(vpb + (long long)j * D + col);
                } else {
                    kst[i] = ldg_b128(kb + (long long)(j - p.prev_rows) * D + col);
                    vst[i] = ldg_b128(vb + (long long)(j - p.prev_rows) * D + col);
                }
            }
        }
    };
    // phi in fp32, z accumulation, hi/lo split, row-major stores into LDS
    auto store_tile = [&](int it, int buf) {
        lds_u16* Vd = smem + buf * BUF;
        lds_u16* Hd = Vd + VT;
        lds_u16* Ld = Hd + FT;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tid + i * NW * 64;
            if (CHUNKS % (NW * 64) == 0 || c < CHUNKS) {
                const int r = c / (D / 8);
                const int col = (c % (D / 8)) * 8;
                const bool valid = j0 + it * BN + r < j1;
                float x[8];
                unpack8(kst[i], x);
                float f[PHI == kPhiPoly2 ? 16 : 8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    f[e] = valid ? elu1(x[e]) : 0.0f;
                    if (PHI == kPhiPoly2) f[8 + e] = valid ? x[e] * x[e] : 0.0f;
                }
#pragma unroll
                for (int e = 0; e < (PHI == kPhiPoly2 ? 16 : 8); ++e) zacc[i][e] += f[e];
#pragma unroll
                for (int half = 0; half < (PHI == kPhiPoly2 ? 2 : 1); ++half) {
                    u32x4 whi, wlo;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float a = f[8 * half + 2 * e], b = f[8 * half + 2 * e + 1];
                        const float ha = round_bf16(a), hb = round_bf16(b);
                        whi[e] = pack2_bf16(ha, hb);
                        wlo[e] = pack2_bf16(a - ha, b - hb);
                    }
                    lds_write_b128(Hd, r * FP + half * D + col, whi);
                    lds_write_b128(Ld, r * FP + half * D + col, wlo);
                }
                u32x4 vv = vst[i];
                if (!valid) vv = u32x4{0u, 0u, 0u, 0u};
                lds_write_b128(Vd, r * VP + col, vv);
            }
        }
    };

    const int tr_row = 8 * h + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    if (ntiles > 0) {
        load_tile(0);
        store_tile(0, 0);
        __syncthreads();
    }
    for (int it = 0; it < ntiles; ++it) {
        const int cur = it & 1;
        if (it + 1 < ntiles) load_tile(it + 1);
        const lds_u16* Vs = smem + cur * BUF;
        const lds_u16* Hs = Vs + VT;
        const lds_u16* Ls = Hs + FT;
#pragma unroll
        for (int ks = 0; ks < BN / 16; ++ks) {
            const int row = 16 * ks + tr_row;
#pragma unroll
            for (int i = 0; i < TPW; ++i) {
                const int tix = wave + i * NW;
                if (TILES % NW == 0 || tix < TILES) {
                    const int dt = tix / NT, nt = tix % NT;
                    const int vcol = 32 * dt + tr_col, fcol = 32 * nt + tr_col;
                    const bf16x8 a = cat(lds_read_tr(Vs, row * VP + vcol), lds_read_tr(Vs, (row + 4) * VP + vcol));
                    const bf16x8 bh_ = cat(lds_read_tr(Hs, row * FP + fcol), lds_read_tr(Hs, (row + 4) * FP + fcol));
                    const bf16x8 bl_ = cat(lds_read_tr(Ls, row * FP + fcol), lds_read_tr(Ls, (row + 4) * FP + fcol));
                    acc[i] = mfma32x32x16(a, bh_, acc[i]);
                    acc[i] = mfma32x32x16(a, bl_, acc[i]);
                }
            }
        }
        if (it + 1 < ntiles) store_tile(it + 1, cur ^ 1);
        __syncthreads();
    }

    // S^T partial: C layout, lane column = feature 32nt + lq, rows d = 32dt + (r/4)*8 + 4h + r%4
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int tix = wave + i * NW;
        if (TILES % NW == 0 || tix < TILES) {
            const int dt = tix / NT, nt = tix % NT;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int drow = 32 * dt + (r >> 2) * 8 + 4 * h + (r & 3);
                outp[(long long)drow * DP + 32 * nt + lq] = acc[i][r];
            }
        }
    }
    // z partial: threads with the same column chunk (tid % (D/8)) hold sums over
    // different rows; reduce them through LDS
    constexpr int COLS = D / 8;
    constexpr int ZW = PHI == kPhiPoly2 ? 16 : 8;
#pragma unroll
    for (int half = 0; half < ZW / 8; ++half) {
        float part[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            part[e] = 0.0f;
#pragma unroll
            for (int i = 0; i < CPT; ++i) part[e] += zacc[i][8 * half + e];
            zred[tid][e] = part[e];
        }
        __syncthreads();
        if (tid < COLS) {
            float s[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) s[e] = 0.0f;
            for (int r = tid; r < NW * 64; r += COLS)
#pragma unroll
                for (int e = 0; e < 8; ++e) s[e] += zred[r][e];
#pragma unroll
            for (int e = 0; e < 8; ++e) outp[D * DP + half * D + 8 * tid + e] = s[e];
        }
        __syncthreads();
    }
}

template <int D>
hipError_t launch_d(const StateParams& p, hipStream_t s) {
    const int blocks = p.BH * p.n_blocks * p.n_sub;
    if (blocks <= 0) return hipSuccess;
    switch (p.phi) {
    case kPhiElu1: state_bf16_kernel<D, kPhiElu1><<<blocks, 256, 0, s>>>(p); break;
    case kPhiPoly2: state_bf16_kernel<D, kPhiPoly2><<<blocks, 256, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_state_bf16(const StateParams& p, hipStream_t s) {
    switch (p.d) {
    case 32: return launch_d<32>(p, s);
    case 64: return launch_d<64>(p, s);
    case 128: return launch_d<128>(p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace rehyat
