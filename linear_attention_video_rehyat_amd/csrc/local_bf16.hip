// local_bf16.hip -- local-softmax + fused hybrid combine kernel, bf16 in/out,
// fp32 accumulation, bf16 MFMA (v_mfma_f32_32x32x16_bf16) on gfx950.
//
// Implements, for every query i of chunk t (ReHyAt, arXiv 2601.04342):
//   softmax branch over the window W_t = frames [max(t T_c - T_o, 0), min((t+1) T_c, F))
//   (the softmax set of the §3.3 equation), computed flash-style with an
//   online max so no N x N score matrix is ever formed;
//   linear branch a^L = phi(q)^T S_t, n^L = phi(q).z_t with the carried state of
//   the keys before the window (§3.1 cached sums, §3.3 linear set);
//   joint normalisation y = (a^S + a^L) / (n^S + n^L) (§3.2, first equation),
//   evaluated in a max-shifted form that is exact and cannot overflow fp32.
//
// Work decomposition: one workgroup of NW waves handles BM = NW*QB*32 query
// rows of one (b, h, chunk); each wave owns QB blocks of 32 queries.  Scores
// are formed transposed, S^T = K Q^T, so that every lane holds one query and
// 16 of its keys: row max and row sum need only in-lane work plus one swap
// between the two 32-lane halves.  P^T then feeds O^T += V^T P^T directly from
// registers; V^T fragments come from the row-major V tile in LDS through the
// transposing LDS read.  K/V tiles of BN keys are double-buffered in LDS.
#include "common.h"
#include "kernels.h"

namespace rehyat {

namespace {

constexpr float kRescaleThreshold = 8.0f;  // log2 units: keep a stale max while P <= 2^8

template <int D, int QB, int NW, int BN, int PHI>
__global__ __launch_bounds__(NW * 64) void local_bf16_kernel(LocalParams p) {
    constexpr int PITCH = D + 8;                 // LDS row pitch (elements), 16-byte aligned rows
    constexpr int TILE = BN * PITCH;
    constexpr int KS = D / 16;                   // k-steps over head_dim
    constexpr int DT = D / 32;                   // 32-row tiles over head_dim
    constexpr int KT = BN / 32;                  // 32-key tiles per LDS tile
    constexpr int BM = NW * QB * 32;
    constexpr int DP = PHI == kPhiPoly2 ? 2 * D : D;
    constexpr int KSL = DP / 16;                 // k-steps over the feature dimension
    constexpr int CHUNKS = BN * D / 8;           // 16-byte chunks per K (or V) tile
    constexpr int CPT = (CHUNKS + NW * 64 - 1) / (NW * 64);

    __shared__ __attribute__((aligned(16))) uint16_t smem_raw[4 * TILE];
    lds_u16* smem = (lds_u16*)smem_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h = lane >> 5;
    const int lq = lane & 31;

    const int item = xcd_remap(blockIdx.x, gridDim.x);
    const int per_bh = p.n_chunks * p.tiles_per_chunk;
    const int bh = item / per_bh;
    const int rem = item - bh * per_bh;
    const int t = rem / p.tiles_per_chunk;
    const int tile = rem - t * p.tiles_per_chunk;
    const int f0 = t * p.Tc;
    const int f1 = min(f0 + p.Tc, p.F);
    const int q_end = f1 * p.HW;
    const int q_start = f0 * p.HW + tile * BM;
    if (q_start >= q_end) return;
    const int w0 = max(f0 - p.To, 0) * p.HW;
    const int nkeys = p.prev_rows + (q_end - w0);

    const uint16_t* qb_ptr = (const uint16_t*)p.q + bh * p.bh_stride;
    const uint16_t* kb_ptr = (const uint16_t*)p.k + bh * p.bh_stride;
    const uint16_t* vb_ptr = (const uint16_t*)p.v + bh * p.bh_stride;
    const int seg_shift = w0 - p.prev_rows;     // virtual key j >= prev_rows is clip row j + seg_shift
    const uint16_t* kp_ptr = p.kp ? (const uint16_t*)p.kp + bh * p.prev_bh_stride : nullptr;
    const uint16_t* vp_ptr = p.vp ? (const uint16_t*)p.vp + bh * p.prev_bh_stride : nullptr;

    // ---- queries: B operand of S^T = K Q^T, held in registers for the whole pass
    bf16x8 qreg[QB][KS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = min(q_start + (wave * QB + qb) * 32 + lq, q_end - 1);
        const uint16_t* src = qb_ptr + (long long)row * D + 8 * h;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qreg[qb][ks] = __builtin_bit_cast(bf16x8, ldg_b128(src + 16 * ks));
    }

    // ---- K/V tile staging: global -> registers -> LDS
    u32x4 kst[CPT], vst[CPT];
    auto load_tile = [&](int it) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tid + i * NW * 64;
            if (CHUNKS % (NW * 64) == 0 || c < CHUNKS) {
                const int r = c / (D / 8);
                const int col = (c % (D / 8)) * 8;
                const int j = min(it * BN + r, nkeys - 1);
                const uint16_t* ks_;
                const uint16_t* vs_;
                if (j < p.prev_rows) {
                    ks_ = kp_ptr + (long long)j * D + col;
                    vs_ = vp_ptr + (long long)j * D + col;
                } else {
                    ks_ = kb_ptr + (long long)(j + seg_shift) * D + col;
                    vs_ = vb_ptr + (long long)(j + seg_shift) * D + col;
                }
                kst[i] = ldg_b128(ks_);
                vst[i] = ldg_b128(vs_);
            }
        }
    };
    auto store_tile = [&](int buf) {
        lds_u16* Kd = smem + buf * 2 * TILE;
        lds_u16* Vd = Kd + TILE;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tid + i * NW * 64;
            if (CHUNKS % (NW * 64) == 0 || c < CHUNKS) {
                const int r = c / (D / 8);
                const int col = (c % (D / 8)) * 8;
                lds_write_b128(Kd, r * PITCH + col, kst[i]);
                lds_write_b128(Vd, r * PITCH + col, vst[i]);
            }
        }
    };

    f32x16 oacc[QB][DT];
    float m2[QB], msum[QB], mtrue[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[qb][dt] = f32x16{};
        m2[qb] = -INFINITY;
        msum[qb] = 0.0f;
        mtrue[qb] = -INFINITY;
    }

    const int ntiles = (nkeys + BN - 1) / BN;
    load_tile(0);
    store_tile(0);
    __syncthreads();

    // V^T fragment addressing for the transposing read (see lds_read_tr)
    const int tr_row = 4 * h + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    for (int it = 0; it < ntiles; ++it) {
        const int cur = it & 1;
        if (it + 1 < ntiles) load_tile(it + 1);
        const lds_u16* Ks = smem + cur * 2 * TILE;
        const lds_u16* Vs = Ks + TILE;

        // S^T = K Q^T: lane holds query lq of each block, keys (r/4)*8 + 4h + r%4
        f32x16 sacc[QB][KT];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) sacc[qb][kt] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
                const bf16x8 a = lds_read_b128(Ks, (32 * kt + lq) * PITCH + 16 * ks + 8 * h);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) sacc[qb][kt] = mfma32x32x16(a, qreg[qb][ks], sacc[qb][kt]);
            }
        }

        // keys past the window end (last tile only)
        if ((it + 1) * BN > nkeys) {
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = it * BN + 32 * kt + (r >> 2) * 8 + 4 * h + (r & 3);
                    if (key >= nkeys) {
#pragma unroll
                        for (int qb = 0; qb < QB; ++qb) sacc[qb][kt][r] = -INFINITY;
                    }
                }
        }

        // online softmax, log2 domain; the running max is only moved when a
        // new score exceeds it by more than kRescaleThreshold
        float mt[QB];
        bool need = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float m = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) m = fmaxf(m, sacc[qb][kt][r]);
            m = xhalf_max(m);
            mtrue[qb] = fmaxf(mtrue[qb], m);
            mt[qb] = m * kLog2e;
            need |= mt[qb] > m2[qb] + kRescaleThreshold;
        }
        if (__any(need)) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const float mn = fmaxf(m2[qb], mt[qb]);
                const float alpha = __builtin_amdgcn_exp2f(m2[qb] - mn);
                msum[qb] *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) oacc[qb][dt] *= alpha;
                m2[qb] = mn;
            }
        }
        bf16x8 pfrag[QB][KT][2];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float negm = -m2[qb];
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int sp = 0; sp < 2; ++sp) {
                    float e[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        e[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[qb][kt][8 * sp + j], kLog2e, negm));
                        msum[qb] += e[j];
                    }
                    u32x4 w;
#pragma unroll
                    for (int j = 0; j < 4; ++j) w[j] = pack2_bf16(e[2 * j], e[2 * j + 1]);
                    pfrag[qb][kt][sp] = __builtin_bit_cast(bf16x8, w);
                }
        }

        // O^T += V^T P^T
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int sp = 0; sp < 2; ++sp) {
                const int row = 32 * kt + 16 * sp + tr_row;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const int col = 32 * dt + tr_col;
                    const bf16x8 a = cat(lds_read_tr(Vs, row * PITCH + col), lds_read_tr(Vs, (row + 8) * PITCH + col));
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) oacc[qb][dt] = mfma32x32x16(a, pfrag[qb][kt][sp], oacc[qb][dt]);
                }
            }

        if (it + 1 < ntiles) store_tile(cur ^ 1);
        __syncthreads();
    }

    // ---------------------------------------------------------------- epilogue
    const bool lin = PHI != kPhiNone && (p.lin_always || w0 > 0);
    const uint16_t* shi = nullptr;
    const uint16_t* slo = nullptr;
    const float* zp = nullptr;
    if (lin) {
        shi = (const uint16_t*)p.s_hi + bh * p.s_bh_stride + t * p.s_chunk_stride;
        slo = (const uint16_t*)p.s_lo + bh * p.s_bh_stride + t * p.s_chunk_stride;
        zp = p.z + bh * p.z_bh_stride + t * p.z_chunk_stride;
    }
    uint16_t* ob_ptr = (uint16_t*)p.out + bh * p.bh_stride;

#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float lsum = xhalf_sum(msum[qb]);
        f32x16 lacc[DT];
        float nl = 0.0f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) lacc[dt] = f32x16{};
        if (PHI != kPhiNone && lin) {
            // a^L^T = S_t^T phi(Q)^T with a three-pass bf16 split of both operands;
            // n^L = phi(q).z in fp32
            float nlp = 0.0f;
#pragma unroll
            for (int ksl = 0; ksl < KSL; ++ksl) {
                float x[8];
                unpack8(__builtin_bit_cast(u32x4, qreg[qb][ksl % KS]), x);
                float f[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) f[j] = ksl < KS ? elu1(x[j]) : x[j] * x[j];
                const f32x4 z0 = *(const f32x4*)(zp + 16 * ksl + 8 * h);
                const f32x4 z1 = *(const f32x4*)(zp + 16 * ksl + 8 * h + 4);
#pragma unroll
                for (int j = 0; j < 4; ++j) nlp += f[j] * z0[j] + f[4 + j] * z1[j];
                u32x4 whi, wlo;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float h0 = round_bf16(f[2 * j]), h1 = round_bf16(f[2 * j + 1]);
                    whi[j] = pack2_bf16(h0, h1);
                    wlo[j] = pack2_bf16(f[2 * j] - h0, f[2 * j + 1] - h1);
                }
                const bf16x8 fhi = __builtin_bit_cast(bf16x8, whi);
                const bf16x8 flo = __builtin_bit_cast(bf16x8, wlo);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const long long off = (long long)(32 * dt + lq) * DP + 16 * ksl + 8 * h;
                    const bf16x8 ahi = __builtin_bit_cast(bf16x8, ldg_b128(shi + off));
                    const bf16x8 alo = __builtin_bit_cast(bf16x8, ldg_b128(slo + off));
                    lacc[dt] = mfma32x32x16(ahi, fhi, lacc[dt]);
                    lacc[dt] = mfma32x32x16(alo, fhi, lacc[dt]);
                    lacc[dt] = mfma32x32x16(ahi, flo, lacc[dt]);
                }
            }
            nl = xhalf_sum(nlp);
        }
        // joint normalisation, shifted by M2 = max(m2, log2 n^L)
        float cs = 1.0f, cl = 0.0f;
        if (PHI != kPhiNone && lin && nl > 0.0f) {
            const float M2 = fmaxf(m2[qb], __builtin_amdgcn_logf(nl));
            cs = __builtin_amdgcn_exp2f(m2[qb] - M2);
            cl = __builtin_amdgcn_exp2f(-M2);
        }
        const float inv = 1.0f / (cs * lsum + cl * nl);

        const int row = q_start + (wave * QB + qb) * 32 + lq;
        const bool valid = row < q_end;
        if (!valid) {
            // rows past the chunk end hold duplicated queries; nothing to store
        } else if (p.pm == nullptr && p.poS == nullptr && p.poL == nullptr && p.pnt == nullptr && p.pnL == nullptr) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float y[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float num = PHI != kPhiNone ? cs * oacc[qb][dt][4 * g + j] + cl * lacc[dt][4 * g + j]
                                                          : oacc[qb][dt][4 * g + j];
                        y[j] = num * inv;
                    }
                    u32x2 w = {pack2_bf16(y[0], y[1]), pack2_bf16(y[2], y[3])};
                    *(u32x2*)(ob_ptr + (long long)row * D + 32 * dt + 8 * g + 4 * h) = w;
                }
        } else {
            const long long prow = bh * (long long)(p.bh_stride / D) + row;
            if (h == 0) {
                if (p.pm) p.pm[prow] = mtrue[qb];
                if (p.pnt) p.pnt[prow] = lsum * __builtin_amdgcn_exp2f(m2[qb] - mtrue[qb] * kLog2e);
                if (p.pnL) p.pnL[prow] = nl;
            }
            const float invl = 1.0f / lsum;
            const float invn = nl > 0.0f ? 1.0f / nl : 0.0f;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int col = 32 * dt + 8 * g + 4 * h;
                    if (p.poS) {
                        f32x4 w = {oacc[qb][dt][4 * g] * invl, oacc[qb][dt][4 * g + 1] * invl,
                                   oacc[qb][dt][4 * g + 2] * invl, oacc[qb][dt][4 * g + 3] * invl};
                        *(f32x4*)(p.poS + prow * D + col) = w;
                    }
                    if (p.poL) {
                        f32x4 w = {lacc[dt][4 * g] * invn, lacc[dt][4 * g + 1] * invn,
                                   lacc[dt][4 * g + 2] * invn, lacc[dt][4 * g + 3] * invn};
                        *(f32x4*)(p.poL + prow * D + col) = w;
                    }
                }
        }
    }
}

template <int D, int QB, int NW, int BN>
hipError_t launch_d(const LocalParams& p, hipStream_t s) {
    const int blocks = p.BH * p.n_chunks * p.tiles_per_chunk;
    if (blocks <= 0) return hipSuccess;
    dim3 grid(blocks), block(NW * 64);
    switch (p.phi) {
    case kPhiNone: local_bf16_kernel<D, QB, NW, BN, kPhiNone><<<grid, block, 0, s>>>(p); break;
    case kPhiElu1: local_bf16_kernel<D, QB, NW, BN, kPhiElu1><<<grid, block, 0, s>>>(p); break;
    case kPhiPoly2: local_bf16_kernel<D, QB, NW, BN, kPhiPoly2><<<grid, block, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Tile configuration: QB query blocks of 32 per wave, NW waves, BN keys per LDS tile.
constexpr int kQB = 2, kNW = 4, kBN = 32;

}  // namespace

int local_bf16_tile_rows(int) { return kQB * kNW * 32; }

hipError_t launch_local_bf16(const LocalParams& p, hipStream_t s) {
    switch (p.d) {
    case 32: return launch_d<32, kQB, kNW, kBN>(p, s);
    case 64: return launch_d<64, kQB, kNW, kBN>(p, s);
    case 128: return launch_d<128, kQB, kNW, kBN>(p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace rehyat
