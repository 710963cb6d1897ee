// f32.hip -- fp32 path of librehyat: the same computation as the bf16 kernels
// (ReHyAt, arXiv 2601.04342: §3.3 partition, §3.1 linear sums, §3.2 joint
// normalisation) on the vector ALU in fp32.  The MI355X fp32 MFMA rate is no
// higher than its fp32 vector rate, so these kernels keep the simple one-query-
// per-lane form with K/V tiles broadcast from LDS.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace rehyat {

namespace {

constexpr int kF32Rows = 128;  // queries per workgroup (one per lane)

template <int D, int PHI>
__global__ __launch_bounds__(kF32Rows) void local_f32_kernel(LocalParams p) {
    constexpr int BN = 32;
    constexpr int DP = PHI == kPhiElu1 ? D : 2 * D;
    __shared__ __attribute__((aligned(16))) float Ks[BN][D];
    __shared__ __attribute__((aligned(16))) float Vs[BN][D];

    const int tid = threadIdx.x;
    const int item = xcd_remap(blockIdx.x, gridDim.x);
    const int per_bh = p.n_chunks * p.tiles_per_chunk;
    const int bh = item / per_bh;
    const int rem = item - bh * per_bh;
    const int t = rem / p.tiles_per_chunk;
    const int tile = rem - t * p.tiles_per_chunk;
    const int f0 = t * p.Tc;
    const int f1 = min(f0 + p.Tc, p.F);
    const int q_end = f1 * p.HW;
    const int q_start = f0 * p.HW + tile * kF32Rows;
    if (q_start >= q_end) return;
    const int w0 = max(f0 - p.To, 0) * p.HW;
    const int nkeys = p.prev_rows + (q_end - w0);
    const int seg_shift = w0 - p.prev_rows;

    const float* qb = (const float*)p.q + bh * p.bh_stride;
    const float* kb = (const float*)p.k + bh * p.bh_stride;
    const float* vb = (const float*)p.v + bh * p.bh_stride;
    const float* kpb = p.kp ? (const float*)p.kp + bh * p.prev_bh_stride : nullptr;
    const float* vpb = p.vp ? (const float*)p.vp + bh * p.prev_bh_stride : nullptr;

    const int row = q_start + tid;
    const bool valid = row < q_end;
    const int rowc = min(row, q_end - 1);
    float q[D], o[D];
#pragma unroll
    for (int c = 0; c < D; ++c) {
        q[c] = qb[(long long)rowc * D + c];
        o[c] = 0.0f;
    }
    float m = -INFINITY, l = 0.0f;

    const int ntiles = (nkeys + BN - 1) / BN;
    for (int it = 0; it < ntiles; ++it) {
        for (int c4 = tid; c4 < BN * D / 4; c4 += kF32Rows) {
            const int r = c4 / (D / 4);
            const int col = (c4 % (D / 4)) * 4;
            const int j = min(it * BN + r, nkeys - 1);
            const float* ks = j < p.prev_rows ? kpb + (long long)j * D : kb + (long long)(j + seg_shift) * D;
            const float* vs = j < p.prev_rows ? vpb + (long long)j * D : vb + (long long)(j + seg_shift) * D;
            *(f32x4*)&Ks[r][col] = *(const f32x4*)(ks + col);
            *(f32x4*)&Vs[r][col] = *(const f32x4*)(vs + col);
        }
        __syncthreads();
        float s[BN];
        float tmax = -INFINITY;
#pragma unroll
        for (int j = 0; j < BN; ++j) {
            float acc = 0.0f;
#pragma unroll
            for (int c = 0; c < D; ++c) acc = fmaf(q[c], Ks[j][c], acc);
            s[j] = it * BN + j < nkeys ? acc : -INFINITY;
            tmax = fmaxf(tmax, s[j]);
        }
        const float mn = fmaxf(m, tmax);
        const float alpha = expf(m - mn);
        l *= alpha;
#pragma unroll
        for (int c = 0; c < D; ++c) o[c] *= alpha;
        m = mn;
#pragma unroll
        for (int j = 0; j < BN; ++j) {
            const float e = expf(s[j] - m);
            l += e;
#pragma unroll
            for (int c = 0; c < D; ++c) o[c] = fmaf(e, Vs[j][c], o[c]);
        }
        __syncthreads();
    }

    // linear branch from the prepared fp32 state S^T [D][DP], z [DP]
    const bool lin = PHI != kPhiNone && (p.lin_always || w0 > 0);
    float al[D];
    float nl = 0.0f;
#pragma unroll
    for (int c = 0; c < D; ++c) al[c] = 0.0f;
    if (PHI != kPhiNone && lin) {
        const float* st = (const float*)p.s_hi + bh * p.s_bh_stride + t * p.s_chunk_stride;
        const float* zp = p.z + bh * p.z_bh_stride + t * p.z_chunk_stride;
        const float* fqr = PHI == kPhiFeat ? (const float*)p.fq + bh * p.fq_bh_stride + (long long)rowc * DP : nullptr;
        for (int c = 0; c < DP; ++c) {
            const float x = q[c % D];
            const float f = PHI == kPhiFeat ? fqr[c] : (c < D ? (x > 0.0f ? x + 1.0f : expf(x)) : x * x);
            nl = fmaf(f, zp[c], nl);
#pragma unroll
            for (int dd = 0; dd < D; ++dd) al[dd] = fmaf(f, st[(long long)dd * DP + c], al[dd]);
        }
    }
    if (!valid) return;
    float cs = 1.0f, cl = 0.0f, M = m;
    if (PHI != kPhiNone && lin && nl > 0.0f) {
        M = fmaxf(m, logf(nl));
        cs = expf(m - M);
        cl = expf(-M);
    }
    const float den = cs * l + cl * nl;  // (n^S + n^L) e^-M
    const float inv = 1.0f / den;
    const bool partials = p.pm || p.pnt || p.poS || p.poL || p.pnL;
    const long long prow = bh * (long long)(p.bh_stride / D) + row;
    if (p.lse) p.lse[prow] = M + logf(den);
    if (!partials) {
        float* ob = (float*)p.out + bh * p.bh_stride + (long long)row * D;
#pragma unroll
        for (int c = 0; c < D; c += 4) {
            f32x4 w;
#pragma unroll
            for (int j = 0; j < 4; ++j) w[j] = (cs * o[c + j] + cl * al[c + j]) * inv;
            *(f32x4*)(ob + c) = w;
        }
    } else {
        if (p.pm) p.pm[prow] = m;
        if (p.pnt) p.pnt[prow] = l;
        if (p.pnL) p.pnL[prow] = nl;
        const float invl = 1.0f / l, invn = nl > 0.0f ? 1.0f / nl : 0.0f;
#pragma unroll
        for (int c = 0; c < D; ++c) {
            if (p.poS) p.poS[prow * D + c] = o[c] * invl;
            if (p.poL) p.poL[prow * D + c] = al[c] * invn;
        }
    }
}

// GRAD: the backward's gradient sums (row r's phi scaled by exp(-lse_r), its
// z weight dsum_r; the second operand is dy)
template <int D, int PHI, bool GRAD = false>
__global__ __launch_bounds__(256) void state_f32_kernel(StateParams p) {
    constexpr int BN = 32;
    constexpr int DP = PHI == kPhiElu1 ? D : 2 * D;
    constexpr int SE = D * DP;
    constexpr int PER = (SE + 255) / 256;
    __shared__ float Fs[BN][DP];
    __shared__ float Vs[BN][D];
    __shared__ float Zw[BN];

    const int tid = threadIdx.x;
    // block -> (bh, u, sub), as in the bf16 kernel
    const int bh = blockIdx.x / p.items_per_bh;
    int sub = blockIdx.x - bh * p.items_per_bh;
    const BlockPart part = state_part(p);
    int u = 0;
    for (; u < p.n_blocks - 1; ++u) {
        const int n = part_block_subs(part, u);
        if (sub < n) break;
        sub -= n;
    }
    int e0, e1;
    part_block_rows(part, u, e0, e1);
    const int j0 = e0 + sub * p.sub_rows;
    const int j1 = min(j0 + p.sub_rows, e1);
    float* outp = p.partial + ((long long)(bh * p.n_blocks + u) * p.n_sub + sub) * (SE + DP);
    const float* kb = (const float*)p.k + bh * p.bh_stride;
    const float* vb = (const float*)p.v + bh * p.bh_stride;
    const float* kpb = p.kp ? (const float*)p.kp + bh * p.prev_bh_stride : nullptr;
    const float* vpb = p.vp ? (const float*)p.vp + bh * p.prev_bh_stride : nullptr;
    const float* fkb = PHI == kPhiFeat ? (const float*)p.fk + bh * p.fk_bh_stride : nullptr;
    const float* fkpb = PHI == kPhiFeat && p.fkp ? (const float*)p.fkp + bh * p.fkp_bh_stride : nullptr;

    float acc[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = 0.0f;
    float zacc = 0.0f;
    for (int base = j0; base < j1; base += BN) {
        for (int x = tid; x < BN * D; x += 256) {
            const int r = x / D, c = x % D;
            const int j = base + r;
            float kv = 0.0f, vv = 0.0f;
            if (j < j1) {
                const float* ks = j < p.prev_rows ? kpb + (long long)j * D : kb + (long long)(j - p.prev_rows) * D;
                const float* vs = j < p.prev_rows ? vpb + (long long)j * D : vb + (long long)(j - p.prev_rows) * D;
                kv = PHI == kPhiFeat ? 0.0f : ks[c];
                vv = vs[c];
                if (PHI != kPhiFeat) Fs[r][c] = kv > 0.0f ? kv + 1.0f : expf(kv);
                if (PHI == kPhiPoly2) Fs[r][D + c] = kv * kv;
            } else {
                if (PHI != kPhiFeat) Fs[r][c] = 0.0f;
                if (PHI == kPhiPoly2) Fs[r][D + c] = 0.0f;
            }
            Vs[r][c] = vv;
        }
        if (GRAD) {  // scale phi by exp(-lse) per row; z weights dsum
            __syncthreads();
            for (int x = tid; x < BN * DP; x += 256) {
                const int r = x / DP, c = x % DP;
                const int j = min(base + r, j1 - 1);
                Fs[r][c] *= expf(-p.row_lse[bh * (p.bh_stride / D) + j]);
            }
            if (tid < BN) Zw[tid] = p.row_d[bh * (p.bh_stride / D) + min(base + tid, j1 - 1)];
        }
        if (PHI == kPhiFeat) {  // precomputed phi(k) rows
            for (int x = tid; x < BN * DP; x += 256) {
                const int r = x / DP, c = x % DP;
                const int j = base + r;
                float f = 0.0f;
                if (j < j1)
                    f = j < p.prev_rows ? fkpb[(long long)j * DP + c] : fkb[(long long)(j - p.prev_rows) * DP + c];
                Fs[r][c] = f;
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = tid + i * 256;
            if (SE % 256 == 0 || e < SE) {
                const int dd = e / DP, c = e % DP;
                float a = acc[i];
#pragma unroll 8
                for (int r = 0; r < BN; ++r) a = fmaf(Vs[r][dd], Fs[r][c], a);
                acc[i] = a;
            }
        }
        if (tid < DP) {
#pragma unroll 8
            for (int r = 0; r < BN; ++r) zacc += GRAD ? Fs[r][tid] * Zw[r] : Fs[r][tid];
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = tid + i * 256;
        if (SE % 256 == 0 || e < SE) outp[e] = acc[i];
    }
    if (tid < DP) outp[SE + tid] = zacc;
}

template <int D>
hipError_t launch_local_d(const LocalParams& p, hipStream_t s) {
    const int blocks = p.BH * p.n_chunks * p.tiles_per_chunk;
    if (blocks <= 0) return hipSuccess;
    switch (p.phi) {
    case kPhiNone: local_f32_kernel<D, kPhiNone><<<blocks, kF32Rows, 0, s>>>(p); break;
    case kPhiElu1: local_f32_kernel<D, kPhiElu1><<<blocks, kF32Rows, 0, s>>>(p); break;
    case kPhiPoly2: local_f32_kernel<D, kPhiPoly2><<<blocks, kF32Rows, 0, s>>>(p); break;
    case kPhiFeat: local_f32_kernel<D, kPhiFeat><<<blocks, kF32Rows, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int D>
hipError_t launch_state_d(const StateParams& p, hipStream_t s) {
    const int blocks = p.BH * p.items_per_bh;
    if (blocks <= 0) return hipSuccess;
    switch (p.phi) {
    case kPhiElu1:
        if (p.row_lse) state_f32_kernel<D, kPhiElu1, true><<<blocks, 256, 0, s>>>(p);
        else state_f32_kernel<D, kPhiElu1><<<blocks, 256, 0, s>>>(p);
        break;
    case kPhiPoly2:
        if (p.row_lse) state_f32_kernel<D, kPhiPoly2, true><<<blocks, 256, 0, s>>>(p);
        else state_f32_kernel<D, kPhiPoly2><<<blocks, 256, 0, s>>>(p);
        break;
    case kPhiFeat: state_f32_kernel<D, kPhiFeat><<<blocks, 256, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

int local_f32_tile_rows(int) { return kF32Rows; }

hipError_t launch_local_f32(const LocalParams& p, hipStream_t s) {
    switch (p.d) {
    case 16: return launch_local_d<16>(p, s);
    case 32: return launch_local_d<32>(p, s);
    case 64: return launch_local_d<64>(p, s);
    case 128: return launch_local_d<128>(p, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_state_f32(const StateParams& p, hipStream_t s) {
    switch (p.d) {
    case 16: return launch_state_d<16>(p, s);
    case 32: return launch_state_d<32>(p, s);
    case 64: return launch_state_d<64>(p, s);
    case 128: return launch_state_d<128>(p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace rehyat
