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
// transposing LDS read.  K/V tiles of BN keys stream into a ring of LDS stages
// by direct global->LDS buffer loads (no register staging), issued STAGES - 1
// tiles ahead (one in the default two-stage ring); rows are stored unpadded with an XOR swizzle of their 16-byte chunks
// so that both the K fragment reads and the transposing V reads are free of
// bank conflicts.
#include <type_traits>

#include "local_common.h"

namespace rehyat {

namespace {

// One wave's share of the direct global->LDS loads of a K/V tile: op o of the
// wave fills 64 consecutive 16-byte LDS chunk positions of the K tile (ops <
// NINST) or of the V tile.  Virtual key row j < prev_rows reads the overlap
// segment, the others read the clip at row j + seg_shift.  Rows past a
// buffer's end read as zero.
template <int NW, int OPW, int OPS, int NINST, int KTILE, int BN, bool PLAIN>
__device__ __forceinline__ void issue_tile_dma(lds_u16* base, int wave, int tile_idx, int prev_rows, int seg_shift,
                                               int rb, const int* op_row, const int* op_c16,
                                               __amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs,
                                               __amdgpu_buffer_rsrc_t kprs, __amdgpu_buffer_rsrc_t vprs) {
    // SEG: 0 every row of the tile lies in the clip, 1 every row in the overlap
    // segment, 2 the tile straddles the two (chosen row by row)
    auto issue = [&](auto seg_c) {
        constexpr int SEG = decltype(seg_c)::value;
#pragma unroll
        for (int o = 0; o < OPW; ++o) {
            const int op = wave + o * NW;
            if (OPS % NW == 0 || op < OPS) {
                // K or V: decided at compile time when the ops split evenly over the waves
                const bool isv = NINST % NW == 0 ? o >= NINST / NW : op >= NINST;
                lds_u16* dst = base + (isv ? KTILE : 0) + 64 * (op % NINST) * 8;
                const int j = tile_idx * BN + op_row[o];  // virtual key row
                const int off_prev = j * rb + op_c16[o];
                const int off_clip = (j + seg_shift) * rb + op_c16[o];
                auto* lds = (__attribute__((address_space(3))) void*)dst;
                if (SEG == 0) {
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(isv ? vrs : krs, lds, 16, off_clip, 0, 0, 0);
                } else if (SEG == 1) {
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(isv ? vprs : kprs, lds, 16, off_prev, 0, 0, 0);
                } else if (isv) {
                    if (j < prev_rows) __builtin_amdgcn_raw_ptr_buffer_load_lds(vprs, lds, 16, off_prev, 0, 0, 0);
                    else __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, lds, 16, off_clip, 0, 0, 0);
                } else {
                    if (j < prev_rows) __builtin_amdgcn_raw_ptr_buffer_load_lds(kprs, lds, 16, off_prev, 0, 0, 0);
                    else __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, lds, 16, off_clip, 0, 0, 0);
                }
            }
        }
    };
    const int t0 = tile_idx * BN;  // first virtual key row of the tile (uniform)
    if (PLAIN || t0 >= prev_rows) issue(std::integral_constant<int, 0>{});
    else if (t0 + BN <= prev_rows) issue(std::integral_constant<int, 1>{});
    else issue(std::integral_constant<int, 2>{});
}

// PLAIN: a whole-clip launch that only stores out (no overlap segment, no lse,
// fp32 copy or partials); its instance carries none of that code.
template <int D, int QB, int NW, int BN, int PHI, int LSTAGES, bool PLAIN>
__global__ __launch_bounds__(NW * 64) void local_bf16_kernel(LocalParams p) {
    constexpr int C = D / 8;                     // 16-byte chunks per row
    constexpr int KTILE = BN * D;                // elements of one K (or V) tile
    constexpr int STAGE = 2 * KTILE;             // one K + one V tile
    constexpr int STAGES = LSTAGES;              // LDS ring; tiles are loaded STAGES-1 ahead
    static_assert(STAGES >= 2 && STAGES <= 4, "2..4 LDS stages");
    constexpr int KS = D / 16;                   // k-steps over head_dim
    constexpr int DT = D / 32;                   // 32-row tiles over head_dim
    constexpr int KT = BN / 32;                  // 32-key tiles per LDS tile
    constexpr int BM = NW * QB * 32;
    constexpr int NINST = BN * C / 64;           // 64-lane DMA instructions per K (or V) tile
    constexpr int OPS = 2 * NINST;               // per tile, K and V
    constexpr int OPW = (OPS + NW - 1) / NW;     // per wave
    static_assert(NINST >= 1, "tile too small");

    __shared__ __attribute__((aligned(16))) uint16_t smem_raw[STAGES * STAGE];
    lds_u16* smem = (lds_u16*)smem_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
    const int h = lane >> 5;
    const int lq = lane & 31;

    // block -> (bh, chunk, query tile); integer division is expanded on the
    // vector ALU, so pin the (uniform) results to scalar registers
    const int item = __builtin_amdgcn_readfirstlane(local_work_item(p, blockIdx.x, gridDim.x, BN));
    const int per_bh = p.n_chunks * p.tiles_per_chunk;
    const int bh = __builtin_amdgcn_readfirstlane(item / per_bh);
    const int rem = item - bh * per_bh;
    const int t = __builtin_amdgcn_readfirstlane(rem / p.tiles_per_chunk);
    const int tile = rem - t * p.tiles_per_chunk;
    const int f0 = t * p.Tc;
    const int f1 = min(f0 + p.Tc, p.F);
    const int q_end = f1 * p.HW;
    const int q_start = f0 * p.HW + tile * BM;
    if (q_start >= q_end) return;
    const int w0 = max(f0 - p.To, 0) * p.HW;
    const int prev_rows = PLAIN ? 0 : p.prev_rows;
    const int nkeys = prev_rows + (q_end - w0);

    const uint16_t* qb_ptr = (const uint16_t*)p.q + bh * p.bh_stride;
    const uint16_t* kb_ptr = (const uint16_t*)p.k + bh * p.bh_stride;
    const uint16_t* vb_ptr = (const uint16_t*)p.v + bh * p.bh_stride;
    const int seg_shift = w0 - prev_rows;     // virtual key j >= prev_rows is clip row j + seg_shift
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

    // ---- K/V tiles: direct global->LDS loads into a ring of STAGES stages.
    // Instruction i of a tile covers physical 16-byte chunk positions
    // 64i .. 64i+63 (1 KB of LDS); lane l fills position P = 64i + l, i.e. row
    // P / C, physical chunk P % C, which holds logical chunk (P % C) ^ swz(row).
    const int rb = D * 2;  // row bytes
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kb_ptr), (short)0, q_end * rb, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(vb_ptr), (short)0, q_end * rb, 0x00020000);
    const __amdgpu_buffer_rsrc_t kprs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kp_ptr ? kp_ptr : kb_ptr), (short)0, prev_rows * rb, 0x00020000);
    const __amdgpu_buffer_rsrc_t vprs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(vp_ptr ? vp_ptr : vb_ptr), (short)0, prev_rows * rb, 0x00020000);
    int op_row[OPW], op_c16[OPW];
#pragma unroll
    for (int o = 0; o < OPW; ++o) {
        const int op = wave + o * NW;
        const int pos = 64 * (op % NINST) + lane;
        op_row[o] = pos / C;
        op_c16[o] = ((pos % C) ^ swz<C>(pos / C)) * 16;
    }
    auto issue_tile = [&](int tile_idx, int stage) {
        issue_tile_dma<NW, OPW, OPS, NINST, KTILE, BN, PLAIN>(smem + stage * STAGE, wave, tile_idx, prev_rows, seg_shift,
                                                       rb, op_row, op_c16, krs, vrs, kprs, vprs);
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

    // V^T fragment addressing for the transposing read (see lds_read_tr):
    // logical row 4h + (lane%16)/4 (+8), column 16*((lane/16)%2) + 4*(lane%4)
    const int tr_row = 4 * h + ((lane & 15) >> 2);
    const int tr_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);  // within a 32-column tile
    const int tr_sub = 4 * (lane & 1);                                // element offset in the chunk
    // Lane-dependent parts of the fragment addresses.  The swizzle depends on
    // the row index mod 16 only, so the 16- and 32-row steps between fragments
    // become immediate offsets of the LDS reads.
    int voff[DT][2], koff[KS];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        const int c = 4 * dt + tr_chunk;
        voff[dt][0] = tr_row * D + ((c ^ swz<C>(tr_row)) << 3) + tr_sub;
        voff[dt][1] = (tr_row + 8) * D + ((c ^ swz<C>(tr_row + 8)) << 3) + tr_sub;
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) koff[ks] = lq * D + (((2 * ks + h) ^ swz<C>(lq)) << 3);

    const int ntiles = (nkeys + BN - 1) / BN;
    constexpr int PF = STAGES - 1;  // tiles loaded ahead
    for (int tt = 0; tt < PF && tt < ntiles; ++tt) issue_tile(tt, tt);

    bf16x8 pfrag[QB][KT][2];
    // O^T += V^T(tile) P^T
    auto pv = [&](const lds_u16* Vs) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int sp = 0; sp < 2; ++sp) {
                const int r = (32 * kt + 16 * sp) * D;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const bf16x8 a = cat(lds_read_tr(Vs, r + voff[dt][0]), lds_read_tr(Vs, r + voff[dt][1]));
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) oacc[qb][dt] = mfma32x32x16(a, pfrag[qb][kt][sp], oacc[qb][dt]);
                }
            }
    };
    // S^T(tile) = K Q^T (lane holds query lq, keys 32kt + (r/4)*8 + 4h + r%4),
    // then the online softmax -> P(tile), log2 domain; the running max is only
    // moved when a new score exceeds it by more than kRescaleThreshold
    // TAIL: the window's last tile (only there are keys past the window end
    // masked; the other tiles carry no per-score test at all)
    auto scores_softmax = [&](auto tail, int it, const lds_u16* Ks) {
        constexpr bool TAIL = decltype(tail)::value;
        f32x16 sacc[QB][KT];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) sacc[qb][kt] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
                const bf16x8 a = lds_read_b128(Ks, 32 * kt * D + koff[ks]);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) sacc[qb][kt] = mfma32x32x16(a, qreg[qb][ks], sacc[qb][kt]);
            }
        }
        // scheduling hint: keep up to 8 K-fragment reads in flight ahead of the
        // MFMAs that consume them (LDS latency is otherwise exposed per pair)
        {
            constexpr int NR = KS * KT, AH = NR < 8 ? NR : 8;
            __builtin_amdgcn_sched_group_barrier(0x100, AH, 0);  // DS reads
#pragma unroll
            for (int i = 0; i < NR - AH; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, QB * AH, 0);
        }
        if (TAIL) {  // keys past the window end
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
    };

    // One iteration: refill the slot read in the previous iteration, then
    // scores, softmax and PV of tile `it`.  The slot being filled and the slot
    // being read are passed as restrict pointers: they never overlap, and the
    // compiler may then keep the transposing V reads clear of the wait for the
    // loads still in flight (it cannot otherwise tell them apart).
    // the linear branch's prepared state S_t^T ([D][D'], hi and lo parts) is
    // staged in LDS so that the epilogue reads it from there instead of every
    // wave loading it from L2: both parts by the last iteration into the slot
    // no tile needs any more when they fit in one slot, else the hi part then
    // and the lo part into the last tile's slot once every wave is done with it
    const bool lin = PHI != kPhiNone && (p.lin_always || w0 > 0);
    constexpr int DP = PHI == kPhiElu1 ? D : 2 * D;
    constexpr int SPART = D * DP;                       // elements of one part
    constexpr bool STAGE_S = PHI != kPhiNone && SPART <= STAGE;
    constexpr bool S_ONE_SLOT = 2 * SPART <= STAGE;
    const uint16_t* shi = nullptr;
    const uint16_t* slo = nullptr;
    if (STAGE_S && lin) {
        shi = (const uint16_t*)p.s_hi + bh * p.s_bh_stride + t * p.s_chunk_stride;
        slo = (const uint16_t*)p.s_lo + bh * p.s_bh_stride + t * p.s_chunk_stride;
    }
    // waves whose query rows all lie past the chunk end (in the chunk's last,
    // partial tile) only take their share of the loads and the barriers
    const bool active = q_start + wave * QB * 32 < q_end;
    auto iteration = [&](auto tail, int it, lds_u16* __restrict__ fill, const lds_u16* __restrict__ cur) {
        if (it + PF < ntiles)
            issue_tile_dma<NW, OPW, OPS, NINST, KTILE, BN, PLAIN>(fill, wave, it + PF, prev_rows, seg_shift, rb, op_row,
                                                           op_c16, krs, vrs, kprs, vprs);
        else if (STAGE_S && lin && it == ntiles - 1) {
            issue_state_dma<D, DP, NW>(fill, wave, lane, shi);
            if (S_ONE_SLOT) issue_state_dma<D, DP, NW>(fill + SPART, wave, lane, slo);
        }
        if (active) {
            scores_softmax(tail, it, cur);
            pv(cur + KTILE);
        }
    };
    auto step = [&](auto tail, int it) {
        // own loads of tile `it` have landed (tiles it+1 .. it+PF-1 may still be
        // in flight), then every wave's have, and every wave is done with the
        // slot refilled next
        const int ahead = min(PF - 1, ntiles - 1 - it);
        if (ahead >= 2) __builtin_amdgcn_s_waitcnt(vm_wait_imm(2 * OPW));
        else if (ahead == 1) __builtin_amdgcn_s_waitcnt(vm_wait_imm(OPW));
        else __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
        lds_barrier();
        iteration(tail, it, smem + ((it + PF) % STAGES) * STAGE, smem + (it % STAGES) * STAGE);
    };
    // the last tile, the only one that can be partial, is peeled off the loop:
    // its key mask then adds no instructions (nor live registers) to the loop
    for (int it = 0; it < ntiles - 1; ++it) step(std::false_type{}, it);
    if (ntiles > 0) step(std::true_type{}, ntiles - 1);

    // ---------------------------------------------------------------- epilogue
    const lds_u16* s_lds = nullptr;
    const lds_u16* s_lds_lo = nullptr;
    if (STAGE_S && lin) {
        lds_u16* hi_slot = smem + ((ntiles - 1 + PF) % STAGES) * STAGE;
        if constexpr (S_ONE_SLOT) {
            s_lds_lo = hi_slot + SPART;
        } else {
            // every wave is done reading the last tile: its slot takes the lo part
            lds_u16* lo_slot = smem + ((ntiles - 1) % STAGES) * STAGE;
            lds_barrier();
            issue_state_dma<D, DP, NW>(lo_slot, wave, lane, slo);
            s_lds_lo = lo_slot;
        }
        __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));  // own share of the staged state
        lds_barrier();                               // everyone's
        s_lds = hi_slot;
    }
    if (!active) return;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
        finish_query_block<D, PHI, PLAIN>(p, qreg[qb], oacc[qb], msum[qb], m2[qb], mtrue[qb],
                                   q_start + (wave * QB + qb) * 32 + lq, q_end, bh, t, h, lq, lin, s_lds,
                                   s_lds_lo);
}

// Tile configuration: QB query blocks of 32 per wave, NW waves, BN keys per LDS
// tile (overridable at build time for tuning sweeps).
#ifndef REHYAT_LOCAL_QB
#define REHYAT_LOCAL_QB 1
#endif
#ifndef REHYAT_LOCAL_NW
#define REHYAT_LOCAL_NW 8
#endif
#ifndef REHYAT_LOCAL_BN
#define REHYAT_LOCAL_BN 128
#endif
#ifndef REHYAT_LOCAL_STAGES
#define REHYAT_LOCAL_STAGES 2
#endif
constexpr int kQB = REHYAT_LOCAL_QB, kNW = REHYAT_LOCAL_NW, kBN = REHYAT_LOCAL_BN, kStages = REHYAT_LOCAL_STAGES;

template <int D, int QB, int NW, int BN>
hipError_t launch_d(const LocalParams& p, hipStream_t s) {
    const int blocks = p.BH * p.n_chunks * p.tiles_per_chunk;
    if (blocks <= 0) return hipSuccess;
    dim3 grid(blocks), block(NW * 64);
    const bool plain = p.prev_rows == 0 && p.lse == nullptr && p.out_f32 == nullptr && p.pm == nullptr &&
                       p.pnt == nullptr && p.poS == nullptr && p.poL == nullptr && p.pnL == nullptr;
#define REHYAT_LOCAL_LAUNCH(PHI_)                                                                    \
    if (plain) local_bf16_kernel<D, QB, NW, BN, PHI_, kStages, true><<<grid, block, 0, s>>>(p);       \
    else local_bf16_kernel<D, QB, NW, BN, PHI_, kStages, false><<<grid, block, 0, s>>>(p);
    switch (p.phi) {
    case kPhiNone: REHYAT_LOCAL_LAUNCH(kPhiNone) break;
    case kPhiElu1: REHYAT_LOCAL_LAUNCH(kPhiElu1) break;
    case kPhiPoly2: REHYAT_LOCAL_LAUNCH(kPhiPoly2) break;
    case kPhiFeat: REHYAT_LOCAL_LAUNCH(kPhiFeat) break;
    default: return hipErrorInvalidValue;
    }
#undef REHYAT_LOCAL_LAUNCH
    return hipGetLastError();
}


}  // namespace

int local_bf16_tile_rows(int) { return kQB * kNW * 32; }
int local_bf16_key_tile(int) { return kBN; }

hipError_t launch_local_bf16(const LocalParams& p, hipStream_t s) {
    switch (p.d) {
    case 32: return launch_d<32, kQB, kNW, kBN>(p, s);
    case 64: return launch_d<64, kQB, kNW, kBN>(p, s);
    case 128: return launch_d<128, kQB, kNW, kBN>(p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace rehyat
