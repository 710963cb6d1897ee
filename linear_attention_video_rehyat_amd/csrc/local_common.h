// local_common.h -- pieces shared by the bf16 local-softmax kernels: LDS tile
// swizzle, wait-count immediates, and the epilogue that adds the linear branch
// and applies the joint normalisation of ReHyAt (arXiv 2601.04342, §3.2 first
// equation, with the §3.1 cached sums S_t, z_t of the §3.3 linear set).
#pragma once

#include "common.h"
#include "kernels.h"

namespace rehyat {

constexpr float kRescaleThreshold = 8.0f;  // log2 units: keep a stale max while P <= 2^8

// s_waitcnt immediate with expcnt and lgkmcnt at their maxima and vmcnt = 0;
// OR in the wanted vmcnt (low 4 bits in [3:0], high 2 bits in [15:14]).
constexpr unsigned kVmcntBase = 0x0F70;
constexpr unsigned vm_wait_imm(int n) { return kVmcntBase | (unsigned)(n & 15) | ((unsigned)(n >> 4) << 14); }

// XOR swizzle of the 16-byte chunks of row r of an unpadded tile with C chunks
// per row (C = head_dim / 8, or D' / 8).  Chosen so that (a) 16 consecutive rows read at
// one logical chunk hit 16 different 4-bank groups (K fragment reads), and (b)
// 4 consecutive rows read at 4 consecutive logical chunks (a transposing V
// read) land in 4 different 16-bank groups.  It depends on r mod 16 only.
template <int C>
__device__ __forceinline__ int swz(int r) {
    // rows of 16 or more chunks: every row starts in the same 4-bank group
    if constexpr (C >= 16) return 4 * (r & 3) + ((r >> 2) & 3);
    else if constexpr (C == 8) return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
    else return (r >> 2) & 3;
}

// Workgroup barrier that does not drain outstanding global->LDS loads (a
// __syncthreads() would); the compiler-only fences keep LDS accesses on their
// side of it.
__device__ __forceinline__ void lds_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Global->LDS copy of one part (bf16 hi or lo) of the prepared state S_t^T,
// [D][DP] row-major with the 16-byte chunks of row r XOR-swizzled by swz(r),
// spread over the NW waves of a workgroup.
template <int D, int DP, int NW>
__device__ __forceinline__ void issue_state_dma(lds_u16* dst, int wave, int lane, const uint16_t* src) {
    constexpr int CS = DP / 8;                   // 16-byte chunks per row
    constexpr int NI = D * DP * 2 / 1024;        // 1 KB instructions per matrix
    constexpr int PER = (NI + NW - 1) / NW;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, D * DP * 2, 0x00020000);
#pragma unroll
    for (int o = 0; o < PER; ++o) {
        const int ins = wave + o * NW;
        if (NI % NW == 0 || ins < NI) {
            const int pos = 64 * ins + lane;
            const int r = pos / CS;
            const int off = r * DP * 2 + ((pos % CS) ^ swz<CS>(r)) * 16;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + 512 * ins),
                                                     16, off, 0, 0, 0);
        }
    }
}

// Epilogue for one block of 32 queries (lane: query lq, half h of the keys).
// oacc holds O^T of the softmax branch scaled by 2^-m2 (log2 domain), msum the
// lane's share of the row sum at the same scale.  When `lin`, the linear
// branch a^L = phi(q)^T S_t, n^L = phi(q).z_t is formed with a three-pass bf16
// split of both MFMA operands (S_t comes prepared as bf16 hi + lo parts; a
// precomputed bf16 phi(q) has no lo part, so two passes) and
// n^L in fp32, and the two branches are combined as
//   y = (2^-M2' a^S + 2^-M2 a^L) / (2^-M2' n^S + 2^-M2 n^L),  M2 = max(m2, log2 n^L),
// which equals (a^S + a^L)/(n^S + n^L) exactly and stays finite in fp32.
// Writes y in bf16, or the per-branch partials when any partial buffer is set.
// PLAIN: the launch only stores out (no lse, fp32 copy or partials).
template <int D, int PHI, bool PLAIN = false>
__device__ __forceinline__ void finish_query_block(const LocalParams& p, const bf16x8 (&q)[D / 16],
                                                   const f32x16 (&oacc)[D / 32], float msum, float m2,
                                                   float mtrue, int row, int q_end, int bh, int t, int h,
                                                   int lq, bool lin, const lds_u16* s_lds = nullptr,
                                                   const lds_u16* s_lds_lo = nullptr) {
    constexpr int KS = D / 16, DT = D / 32;
    constexpr bool FEAT = PHI == kPhiFeat;  // phi(q) precomputed in bf16: no lo part
    constexpr int DP = PHI == kPhiElu1 ? D : 2 * D;
    constexpr int KSL = PHI == kPhiNone ? 1 : DP / 16;
    const float lsum = xhalf_sum(msum);
    lin = PHI != kPhiNone && lin;
    // phi(q): n^L in fp32 and the bf16 hi/lo MFMA operands, kept in registers
    // unless there are too many of them (then formed again per output slice);
    // a precomputed phi(q) has no lo part and is always kept
    constexpr bool KEEP = FEAT || KSL <= 8;
    const uint16_t* fqrow =
        FEAT ? (const uint16_t*)p.fq + bh * p.fq_bh_stride + (long long)min(row, q_end - 1) * DP + 8 * h : nullptr;
    auto phi_frag = [&](int ksl, bf16x8& fh, bf16x8& fl, float* f) {
        if constexpr (FEAT) {
            const u32x4 w = ldg_b128(fqrow + 16 * ksl);
            unpack8(w, f);
            fh = __builtin_bit_cast(bf16x8, w);
            fl = bf16x8{};
            return;
        }
        float x[8];
        unpack8(__builtin_bit_cast(u32x4, q[ksl % KS]), x);
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = ksl < KS ? elu1(x[j]) : x[j] * x[j];
        u32x4 whi, wlo;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const u32x2 hl = split2_bf16(f[2 * j], f[2 * j + 1]);
            whi[j] = hl[0];
            wlo[j] = hl[1];
        }
        fh = __builtin_bit_cast(bf16x8, whi);
        fl = __builtin_bit_cast(bf16x8, wlo);
    };
    bf16x8 fhi[KEEP ? KSL : 1], flo[KEEP && !FEAT ? KSL : 1];
    float nl = 0.0f;
    const uint16_t* shi = nullptr;
    const uint16_t* slo = nullptr;
    if (lin) {
        shi = (const uint16_t*)p.s_hi + bh * p.s_bh_stride + t * p.s_chunk_stride;
        slo = (const uint16_t*)p.s_lo + bh * p.s_bh_stride + t * p.s_chunk_stride;
        const float* zp = p.z + bh * p.z_bh_stride + t * p.z_chunk_stride;
        float nlp = 0.0f;
#pragma unroll
        for (int ksl = 0; ksl < KSL; ++ksl) {
            float f[8];
            bf16x8 fh, fl;
            phi_frag(ksl, fh, fl, f);
            if (KEEP) {
                fhi[KEEP ? ksl : 0] = fh;
                if (!FEAT) flo[KEEP && !FEAT ? ksl : 0] = fl;
            }
            const f32x4 z0 = *(const f32x4*)(zp + 16 * ksl + 8 * h);
            const f32x4 z1 = *(const f32x4*)(zp + 16 * ksl + 8 * h + 4);
#pragma unroll
            for (int j = 0; j < 4; ++j) nlp += f[j] * z0[j] + f[4 + j] * z1[j];
        }
        nl = xhalf_sum(nlp);
    }
    float cs = 1.0f, cl = 0.0f, M2 = m2;
    if (lin && nl > 0.0f) {
        M2 = fmaxf(m2, __builtin_amdgcn_logf(nl));
        cs = __builtin_amdgcn_exp2f(m2 - M2);
        cl = __builtin_amdgcn_exp2f(-M2);
    }
    const float den = cs * lsum + cl * nl;  // (n^S + n^L) 2^-M2
    const float inv = 1.0f / den;
    const bool store_out = PLAIN || (p.pm == nullptr && p.poS == nullptr && p.poL == nullptr &&
                                     p.pnt == nullptr && p.pnL == nullptr);
    const bool valid = row < q_end;  // rows past the chunk end hold duplicated queries
    const long long prow = bh * (long long)(p.bh_stride / D) + row;
    if (!PLAIN && p.lse && valid && h == 0) p.lse[prow] = kLn2 * (M2 + __builtin_amdgcn_logf(den));
    if (!PLAIN && !store_out && valid && h == 0) {
        if (p.pm) p.pm[prow] = mtrue;
        if (p.pnt) p.pnt[prow] = lsum * __builtin_amdgcn_exp2f(m2 - mtrue * kLog2e);
        if (p.pnL) p.pnL[prow] = nl;
    }
    const float invl = 1.0f / lsum;
    const float invn = nl > 0.0f ? 1.0f / nl : 0.0f;
    uint16_t* ob_ptr = (uint16_t*)p.out + bh * p.bh_stride;
    // a^L^T = S_t^T phi(Q)^T with a three-pass bf16 split (hi*hi + lo*hi + hi*lo)
    // of both operands.  Fragment (32-column slice dt, 16-feature step ksl) of
    // the staged copies in LDS (DP / 8 chunks per row, by issue_state_dma) or
    // of the prepared state in global memory:
    auto state_frag = [&](int dt, int ksl, bf16x8& ahi, bf16x8& alo) {
        if (s_lds) {
            const int off = (32 * dt + lq) * DP + (((2 * ksl + h) ^ swz<DP / 8>(lq)) << 3);
            ahi = lds_read_b128(s_lds, off);
            alo = lds_read_b128(s_lds_lo, off);
        } else {
            const long long off = (long long)(32 * dt + lq) * DP + 16 * ksl + 8 * h;
            ahi = __builtin_bit_cast(bf16x8, ldg_b128(shi + off));
            alo = __builtin_bit_cast(bf16x8, ldg_b128(slo + off));
        }
    };
    // Without the phi(q) fragments in registers, each 16-feature step's phi is
    // formed once for all four slices, whose accumulators then interleave (each
    // slice still adds its products in the same order).  With them, one slice
    // at a time: the four accumulators at once cost the main loop more than the
    // chains' latency does (measured 1.2 % slower at d = 128).
    f32x16 lall[KEEP ? 1 : DT];
    if constexpr (!KEEP) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) lall[dt] = f32x16{};
        if (lin) {
#pragma unroll
            for (int ksl = 0; ksl < KSL; ++ksl) {
                bf16x8 fh, fl;
                float f[8];
                phi_frag(ksl, fh, fl, f);
                bf16x8 ahi[DT], alo[DT];
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) state_frag(dt, ksl, ahi[dt], alo[dt]);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) lall[dt] = mfma32x32x16(ahi[dt], fh, lall[dt]);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) lall[dt] = mfma32x32x16(alo[dt], fh, lall[dt]);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) lall[dt] = mfma32x32x16(ahi[dt], fl, lall[dt]);
            }
        }
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        f32x16 lacc = f32x16{};
        if constexpr (!KEEP) {
            lacc = lall[dt];
        } else if (lin) {
#pragma unroll
            for (int ksl = 0; ksl < KSL; ++ksl) {
                bf16x8 ahi, alo;
                state_frag(dt, ksl, ahi, alo);
                const bf16x8 fh = fhi[ksl];
                lacc = mfma32x32x16(ahi, fh, lacc);
                lacc = mfma32x32x16(alo, fh, lacc);
                if (!FEAT) lacc = mfma32x32x16(ahi, flo[FEAT ? 0 : ksl], lacc);
            }
        }
        if (!valid) continue;
        if (store_out) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float y[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float num = PHI != kPhiNone ? cs * oacc[dt][4 * g + j] + cl * lacc[4 * g + j]
                                                      : oacc[dt][4 * g + j];
                    y[j] = num * inv;
                }
                u32x2 w = {pack2_bf16(y[0], y[1]), pack2_bf16(y[2], y[3])};
                *(u32x2*)(ob_ptr + (long long)row * D + 32 * dt + 8 * g + 4 * h) = w;
                if (!PLAIN && p.out_f32)
                    *(f32x4*)(p.out_f32 + prow * D + 32 * dt + 8 * g + 4 * h) = f32x4{y[0], y[1], y[2], y[3]};
            }
        } else if constexpr (!PLAIN) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = 32 * dt + 8 * g + 4 * h;
                if (p.poS) {
                    f32x4 w = {oacc[dt][4 * g] * invl, oacc[dt][4 * g + 1] * invl, oacc[dt][4 * g + 2] * invl,
                               oacc[dt][4 * g + 3] * invl};
                    *(f32x4*)(p.poS + prow * D + col) = w;
                }
                if (p.poL) {
                    f32x4 w = {lacc[4 * g] * invn, lacc[4 * g + 1] * invn, lacc[4 * g + 2] * invn,
                               lacc[4 * g + 3] * invn};
                    *(f32x4*)(p.poL + prow * D + col) = w;
                }
            }
        }
    }
}

}  // namespace rehyat
