// state_bf16.hip -- phi-map + block-state kernel (bf16 inputs, fp32 state).
//
// For each block of keys of the state partition (the delta blocks E_u of the
// recurrent form, or the finer blocks of the bidirectional form; see
// state_block_frames) and each contiguous sub-block of it, computes
//   S^T_partial = sum_j v_j phi(k_j)^T   ([head_dim][D'], fp32)
//   z_partial   = sum_j phi(k_j)         ([D'], fp32)
// -- the cached linear-attention sums of ReHyAt §3.1 (arXiv 2601.04342),
// restricted to one block.  The cross-chunk scan adds them up into the state of
// each chunk (the §3.3 linear set is the union of the earlier delta blocks).
//
// K and V tiles of 64 keys stream through a 4-stage LDS ring by direct
// global->LDS loads (three tiles in flight; unpadded rows with XOR-swizzled
// 16-byte chunks).  Eight waves (two per SIMD) share the 32-wide feature tiles
// of D': wave w owns tiles w, w + 8, ...; when D' has fewer tiles than waves,
// the waves sharing one split the 16-key steps and are summed at the end.
// Both MFMA operands are read through the transposing LDS read: A = V^T (32
// head_dim rows x 16 keys), B = phi(K) (16 keys x 32 features); phi is applied
// to the B fragment in registers, in fp32, and split into bf16 hi + lo parts,
// so the products carry ~16 significant bits of phi(k) while v is exact in
// bf16.  z is summed on the vector ALU from the unsplit fp32 values.
// With the learned feature maps (kPhiFeat) phi(k) comes precomputed in bf16:
// the K tile holds phi(k) rows (D' = 2 head_dim columns, a 3-stage ring), its
// transposing reads are the B fragments as they are, one MFMA per output tile.
#include <type_traits>

#include "copy_rows.h"
#include "local_common.h"

namespace rehyat {

namespace {

#ifndef REHYAT_STATE_BN
#define REHYAT_STATE_BN 64
#endif
constexpr int kStateBN = REHYAT_STATE_BN;  // keys per LDS tile

// waves per workgroup: two per SIMD, except when D' is a single 32-wide tile
// (then 4 waves already split the 4 16-key steps of a tile)
constexpr int state_waves(int dp) { return dp / 32 == 1 ? 4 : 8; }
#ifndef REHYAT_STATE_STAGES
#define REHYAT_STATE_STAGES 4
#endif
constexpr int kStateStages = REHYAT_STATE_STAGES;

// Cache policy of the K/V tile loads: nontemporal (the "nt" bit, 2 in the
// intrinsic's cache-policy operand on gfx950).  The pass reads each key once.
// Normal loads allocate in the caches, and where those hold dirty lines (the
// outputs of earlier work) every fill first waits for a write-back: measured
// on the box, a direct-to-LDS stream of the Wan shape's 172 MB of K and V rows
// ran at 2.6 TB/s after 512 MB of writes and at 6.1 TB/s with nt loads (this
// kernel: 72.9 -> 47.2 us after the same writes, 46.9 -> 46.5 us without them).
#ifndef REHYAT_STATE_LOAD_POLICY
#define REHYAT_STATE_LOAD_POLICY 2
#endif
constexpr int kStateLoadPolicy = REHYAT_STATE_LOAD_POLICY;

// One wave's share of the global->LDS loads of a K/V tile (instructions of 1
// KB: the first NK fill the K tile, KW columns wide -- the keys, or their
// precomputed features -- and the next NV the V tile, D columns wide).
// Virtual key j < prev_rows reads the overlap segment, the others read the
// clip at row j - prev_rows.  Rows past a resource's end read as zero.
template <int D, int KW, int BN, int NW, int OPW>
__device__ __forceinline__ void state_load_tile(lds_u16* base, int wave, int lane, int j0, int prev_rows,
                                                __amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs,
                                                __amdgpu_buffer_rsrc_t kprs, __amdgpu_buffer_rsrc_t vprs) {
    constexpr int NK = BN * KW / 512;
#pragma unroll
    for (int o = 0; o < OPW; ++o) {
        const int op = wave + o * NW;
        const bool isv = op >= NK;
        const int ins = isv ? op - NK : op;
        const int pos = 64 * ins + lane;
        const int C = isv ? D / 8 : KW / 8;  // uniform per instruction
        const int r = pos / C;
        const int c16 = ((pos % C) ^ (isv ? swz<D / 8>(r) : swz<KW / 8>(r))) * 16;
        const int rb = isv ? D * 2 : KW * 2;
        const int j = j0 + r;
        auto* lds = (__attribute__((address_space(3))) void*)(base + (isv ? BN * KW : 0) + 64 * 8 * ins);
        if (prev_rows == 0) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(isv ? vrs : krs, lds, 16, j * rb + c16, 0, 0, kStateLoadPolicy);
        } else if (j >= prev_rows) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(isv ? vrs : krs, lds, 16, (j - prev_rows) * rb + c16, 0, 0, kStateLoadPolicy);
        } else {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(isv ? vprs : kprs, lds, 16, j * rb + c16, 0, 0, kStateLoadPolicy);
            asm volatile("");  // keeps the two loads apart (a merged load would need a per-lane resource)
        }
    }
}

// Waves per workgroup for head dim D and feature map PHI (the tile loads must
// split evenly over them).
constexpr int state_nw(int d, int phi) {
    return phi == kPhiFeat && d == 32 ? 4 : state_waves(phi == kPhiElu1 ? d : 2 * d);
}

// GRAD: the backward's gradient sums (rows are queries of a chunk, the second
// operand is dy; row r's phi is scaled by exp(-lse_r) and its z weight is dsum_r)
// One sub-block (work item) of the partition: its partial sums.
template <int D, int PHI, bool GRAD>
__device__ __forceinline__ void state_item(const StateParams& p, const int item) {
    constexpr bool FEAT = PHI == kPhiFeat;            // phi(k) rows come precomputed
    constexpr int DP = PHI == kPhiElu1 ? D : 2 * D;
    constexpr int KW = FEAT ? DP : D;                 // columns of the K tile
    constexpr int NW = state_nw(D, PHI), BN = kStateBN;
    constexpr int NS = FEAT ? 3 : GRAD ? (kStateStages < 4 ? kStateStages : 4) : kStateStages;
    constexpr int NT = DP / 32;                       // 32-wide feature tiles
    constexpr int NTW = NT >= NW ? NT / NW : 1;       // feature tiles per wave
    constexpr int SPLIT = NT >= NW ? 1 : NW / NT;     // waves sharing a feature tile
    constexpr int DT = D / 32;
    constexpr int C = D / 8;
    constexpr int KTILE = BN * KW;                    // elements of the K tile
    constexpr int GROWS = GRAD ? 4 * BN : 0;          // GRAD: the tile's lse, then its dsum (fp32)
    constexpr int STAGE = KTILE + BN * D + GROWS;     // K tile, V tile, per-row values
    constexpr int NLD = (KTILE + BN * D) * 2 / 1024;  // 1 KB load instructions per stage
    constexpr int OPW = NLD / NW;                     // per wave and stage
    constexpr int KSTEPS = BN / 16;
    static_assert(NT % NW == 0 || NW % NT == 0, "feature tiles must split evenly over the waves");
    static_assert(NLD % NW == 0, "tile loads must split evenly over the waves");
    static_assert(KSTEPS % SPLIT == 0, "16-key steps must split evenly over the waves sharing a tile");
    static_assert(NS >= 2 && NS <= 5, "2 to 5 LDS stages");
    static_assert(!GRAD || BN == 64, "one 4-byte-per-lane load carries a tile's lse (and one its dsum)");

    // the ring, reused at the end for the sums of the waves that share a feature
    // tile (one share at a time)
    constexpr int RED_U16 = SPLIT > 1 ? 2 * (NT * DT * 16 * 64 + NT * 32) : 0;
    constexpr int SMEM_U16 = NS * STAGE > RED_U16 ? NS * STAGE : RED_U16;
    __shared__ __attribute__((aligned(16))) uint16_t smem_raw[SMEM_U16];
    lds_u16* const smem = (lds_u16*)smem_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5;
    const int lq = lane & 31;
    const int nt0 = wave % (NT >= NW ? NW : NT);      // first feature tile of the wave
    const int kpart = wave / (NT >= NW ? NW : NT);    // which share of the 16-key steps

    // item -> (bh, u, sub): the sub-blocks of a (b, h), block by block
    const int bh = item / p.items_per_bh;
    int sub = item - bh * p.items_per_bh;
    const BlockPart part = state_part(p);
    int u = 0;
    for (; u < p.n_blocks - 1; ++u) {
        const int n = part_block_subs(part, u);
        if (sub < n) break;
        sub -= n;
    }
    int e0, e1;  // virtual key rows of the block
    part_block_rows(part, u, e0, e1);
    const int j0 = e0 + sub * p.sub_rows;
    const int j1 = min(j0 + p.sub_rows, e1);
    const int nkeys = max(j1 - j0, 0);
    const int ntiles = (nkeys + BN - 1) / BN;
    float* outp = p.partial + ((long long)(bh * p.n_blocks + u) * p.n_sub + sub) * (D * DP + DP);

    // resources end at the block's last row: rows past it read as zero
    const int rb = D * 2, krb = KW * 2;
    const int prev_rows = p.prev_rows;
    const uint16_t* kb = FEAT ? (const uint16_t*)p.fk + bh * p.fk_bh_stride : (const uint16_t*)p.k + bh * p.bh_stride;
    const uint16_t* vb = (const uint16_t*)p.v + bh * p.bh_stride;
    const void* kp = FEAT ? p.fkp : p.kp;
    const uint16_t* kpb = kp ? (const uint16_t*)kp + bh * (FEAT ? p.fkp_bh_stride : p.prev_bh_stride) : kb;
    const uint16_t* vpb = p.vp ? (const uint16_t*)p.vp + bh * p.prev_bh_stride : vb;
    const int clip_rows = max(e1 - prev_rows, 0);
    const int prev_end = min(e1, prev_rows);
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)kb, (short)0, clip_rows * krb, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vb, (short)0, clip_rows * rb, 0x00020000);
    const __amdgpu_buffer_rsrc_t kprs = __builtin_amdgcn_make_buffer_rsrc((void*)kpb, (short)0, prev_end * krb, 0x00020000);
    const __amdgpu_buffer_rsrc_t vprs = __builtin_amdgcn_make_buffer_rsrc((void*)vpb, (short)0, prev_end * rb, 0x00020000);
    // GRAD: rows are the clip's query rows (no overlap segment); waves 0 and 1
    // also bring the tile's lse and dsum into the stage, through the same
    // asynchronous path, so the per-row values never stall the MFMA loop
    const bool grow_wave = GRAD && wave < 2;
    __amdgpu_buffer_rsrc_t grs = krs;
    if constexpr (GRAD) {
        const float* g = (wave == 0 ? p.row_lse : p.row_d) + bh * (p.bh_stride / D);
        grs = __builtin_amdgcn_make_buffer_rsrc((void*)g, (short)0, e1 * 4, 0x00020000);
    }
    auto load_tile = [&](lds_u16* base, int t) {
        state_load_tile<D, KW, BN, NW, OPW>(base, wave, lane, j0 + t * BN, prev_rows, krs, vrs, kprs, vprs);
        if (grow_wave) {
            auto* lds = (__attribute__((address_space(3))) void*)(base + KTILE + BN * D + 2 * BN * wave);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(grs, lds, 4, (j0 + t * BN + lane) * 4, 0, 0, 0);
        }
    };

    // transposing-read addressing (see lds_read_tr): for its column, lane
    // (half h) receives keys 4h..4h+3 of the first read and 8+4h..8+4h+3 of
    // the second; A (V^T) and B (phi(K)) use the same key order.  The swizzle
    // depends on the row mod 16 only, so the 16-key step is an immediate.
    const int tr_row = 4 * h + ((lane & 15) >> 2);
    const int tr_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    const int tr_sub = 4 * (lane & 1);
    int toff[DT][2];  // column block c (32 columns) of a row-major K or V tile
#pragma unroll
    for (int c = 0; c < DT; ++c) {
        const int ch = 4 * c + tr_chunk;
        toff[c][0] = tr_row * D + ((ch ^ swz<C>(tr_row)) << 3) + tr_sub;
        toff[c][1] = (tr_row + 8) * D + ((ch ^ swz<C>(tr_row + 8)) << 3) + tr_sub;
    }
    // the same for the KW-wide feature tile (precomputed phi(k) rows)
    int foff[FEAT ? NTW : 1][2];
    if constexpr (FEAT) {
#pragma unroll
        for (int i = 0; i < NTW; ++i) {
            const int ch = 4 * (nt0 + i * NW) + tr_chunk;
            foff[i][0] = tr_row * KW + ((ch ^ swz<KW / 8>(tr_row)) << 3) + tr_sub;
            foff[i][1] = (tr_row + 8) * KW + ((ch ^ swz<KW / 8>(tr_row + 8)) << 3) + tr_sub;
        }
    }

    f32x16 acc[NTW][DT];
    float zpart[NTW];
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
        zpart[i] = 0.0f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[i][dt] = f32x16{};
    }

    // the wave's 16-key steps of one tile
    // (the tail tile masks keys past the sub-block; full tiles skip the test)
    auto tile_steps = [&](auto tail, int t, const lds_u16* __restrict__ Ks, const lds_u16* __restrict__ Vs) {
        constexpr bool TAIL = decltype(tail)::value;
#pragma unroll
        for (int s = 0; s < KSTEPS / SPLIT; ++s) {
            const int ks = s * SPLIT + kpart;
            const int r16 = 16 * ks * D;
            bf16x8 a[DT];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                a[dt] = cat(lds_read_tr(Vs, r16 + toff[dt][0]), lds_read_tr(Vs, r16 + toff[dt][1]));
            const int kbase = t * BN + 16 * ks + 4 * h;  // key of element 0 (elements 4..7: +8)
            float gc[GRAD ? 8 : 1], gd[GRAD ? 8 : 1];  // per-row scale and z weight (backward)
            if constexpr (GRAD) {
                // the stage's lse (BN floats), then dsum; rows past the block read as zero
                typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
                const lds_f32x4* gv = (const lds_f32x4*)(Vs + BN * D);
                const f32x4 l0 = gv[4 * ks + h], l1 = gv[4 * ks + h + 2];
                const f32x4 d0 = gv[BN / 4 + 4 * ks + h], d1 = gv[BN / 4 + 4 * ks + h + 2];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    gc[e] = __expf(-l0[e]);
                    gc[e + 4] = __expf(-l1[e]);
                    gd[e] = d0[e];
                    gd[e + 4] = d1[e];
                }
            }
            if constexpr (FEAT) {
                // phi(k) is already bf16: one MFMA per output tile, no split
#pragma unroll
                for (int i = 0; i < NTW; ++i) {
                    bf16x8 b = cat(lds_read_tr(Ks, 16 * ks * KW + foff[i][0]), lds_read_tr(Ks, 16 * ks * KW + foff[i][1]));
                    if (TAIL) {
                        u32x4 w = __builtin_bit_cast(u32x4, b);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int key = kbase + (e < 2 ? 2 * e : 2 * e + 4);  // elements 2e, 2e+1
                            const uint32_t lo = key < nkeys ? 0xffffu : 0u, hi = key + 1 < nkeys ? 0xffff0000u : 0u;
                            w[e] &= lo | hi;
                        }
                        b = __builtin_bit_cast(bf16x8, w);
                    }
                    float f[8];
                    unpack8(__builtin_bit_cast(u32x4, b), f);
#pragma unroll
                    for (int e = 0; e < 8; ++e) zpart[i] += f[e];
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) acc[i][dt] = mfma32x32x16(a[dt], b, acc[i][dt]);
                }
                continue;
            }
#pragma unroll
            for (int i = 0; i < NTW; ++i) {
                const int nt = nt0 + i * NW;
                const int kc = (nt % (D / 32));  // K column block the features come from
                const bool square = PHI == kPhiPoly2 && nt >= D / 32;
                const bf16x4 k0 = lds_read_tr(Ks, r16 + toff[kc][0]);
                const bf16x4 k1 = lds_read_tr(Ks, r16 + toff[kc][1]);
                float f[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = (float)(e < 4 ? k0[e] : k1[e - 4]);
                    const int key = kbase + (e < 4 ? e : e + 4);
                    const float y = square ? x * x : elu1(x);
                    f[e] = !TAIL || key < nkeys ? y : 0.0f;
                    if constexpr (GRAD) {
                        f[e] *= gc[e];
                        zpart[i] += f[e] * gd[e];
                    } else {
                        zpart[i] += f[e];
                    }
                }
                u32x4 whi, wlo;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const u32x2 hl = split2_bf16(f[2 * e], f[2 * e + 1]);
                    whi[e] = hl[0];
                    wlo[e] = hl[1];
                }
                const bf16x8 bhi = __builtin_bit_cast(bf16x8, whi), blo = __builtin_bit_cast(bf16x8, wlo);
                // every hi product, then every lo product: consecutive products go to
                // different accumulators, so none waits for the one before it (each
                // accumulator still adds hi, then lo)
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) acc[i][dt] = mfma32x32x16(a[dt], bhi, acc[i][dt]);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) acc[i][dt] = mfma32x32x16(a[dt], blo, acc[i][dt]);
            }
        }
    };
    // the slot being filled and the slot being read never overlap; as restrict
    // pointers they keep the transposing reads clear of a wait for the loads
    auto iteration = [&](auto tail, int t, lds_u16* __restrict__ fill, const lds_u16* __restrict__ cur) {
        if (t + NS - 1 < ntiles) load_tile(fill, t + NS - 1);
        tile_steps(tail, t, cur, cur + KTILE);
    };

    for (int t = 0; t < NS - 1 && t < ntiles; ++t) load_tile(smem + t * STAGE, t);
    // the last tile, the only one that can be partial, is peeled off the loop
    // and alone masks keys past the sub-block: with both forms inside the
    // loop, the two paths left the accumulators in different registers and
    // every iteration copied them back (32 64-bit moves per tile and wave)
    auto step = [&](auto tail, int t) {
        // own loads of tile t have landed (later tiles may be in flight), then
        // every wave's have, and every wave is done with the slot refilled next
        const int ahead = min(NS - 2, ntiles - 1 - t);
        if (GRAD && grow_wave) {  // one more load per stage
            constexpr int PER = OPW + 1;
            if (ahead >= 3) __builtin_amdgcn_s_waitcnt(vm_wait_imm(3 * PER));
            else if (ahead == 2) __builtin_amdgcn_s_waitcnt(vm_wait_imm(2 * PER));
            else if (ahead == 1) __builtin_amdgcn_s_waitcnt(vm_wait_imm(PER));
            else __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
        } else {
            if (ahead >= 3) __builtin_amdgcn_s_waitcnt(vm_wait_imm(3 * OPW));
            else if (ahead == 2) __builtin_amdgcn_s_waitcnt(vm_wait_imm(2 * OPW));
            else if (ahead == 1) __builtin_amdgcn_s_waitcnt(vm_wait_imm(OPW));
            else __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
        }
        lds_barrier();
        iteration(tail, t, smem + ((t + NS - 1) % NS) * STAGE, smem + (t % NS) * STAGE);
    };
    for (int t = 0; t < ntiles - 1; ++t) step(std::false_type{}, t);
    if (ntiles > 0) step(std::true_type{}, ntiles - 1);

    // ---- write the partial: S^T in C layout (column = feature 32nt + lq, row
    // d = 32dt + (r/4)*8 + 4h + r%4), z from the two lane halves; waves that
    // share a feature tile are summed through LDS first
    float z[NTW];
#pragma unroll
    for (int i = 0; i < NTW; ++i) z[i] = xhalf_sum(zpart[i]);
    if (SPLIT > 1) {
        // shares 1, 2, ... added to share 0 in turn through one buffer
        __syncthreads();  // the ring is reused
        float* red = (float*)smem_raw;  // [NT][DT][16][64] + z [NT][32]
        float* zred = red + NT * DT * 16 * 64;
#pragma unroll 1
        for (int sp = 1; sp < SPLIT; ++sp) {
            if (kpart == sp) {
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) red[((nt0 * DT + dt) * 16 + r) * 64 + lane] = acc[0][dt][r];
                if (lane < 32) zred[nt0 * 32 + lq] = z[0];
            }
            __syncthreads();
            if (kpart == 0) {
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[0][dt][r] += red[((nt0 * DT + dt) * 16 + r) * 64 + lane];
                z[0] += lane < 32 ? zred[nt0 * 32 + lq] : 0.0f;
            }
            __syncthreads();
        }
        if (kpart > 0) return;
    }
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
        const int f = 32 * (nt0 + i * NW) + lq;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int drow = 32 * dt + (r >> 2) * 8 + 4 * h + (r & 3);
                outp[(long long)drow * DP + f] = acc[i][dt][r];
            }
        if (lane < 32) outp[(long long)D * DP + f] = z[i];
    }
}

// One workgroup per sub-block, in the XCD-aware order (only the workgroups
// with work are launched).
template <int D, int PHI, bool GRAD = false>
__global__ __launch_bounds__(state_nw(D, PHI) * 64) void state_bf16_kernel(StateParams p) {
    state_item<D, PHI, GRAD>(p, __builtin_amdgcn_readfirstlane(xcd_remap(blockIdx.x, gridDim.x)));
}

// A few workgroups taking the sub-blocks in turn (the streaming fold, which
// runs beside a local-attention launch on the CUs that launch leaves idle: one
// workgroup per idle CU, so that none waits for a CU the local launch holds).
// Each sub-block's partial is computed exactly as above.
template <int D, int PHI>
__global__ __launch_bounds__(state_nw(D, PHI) * 64) void state_bf16_multi_kernel(StateParams p) {
    const int n = p.BH * p.items_per_bh;
    for (int item = blockIdx.x; item < n; item += gridDim.x) {
        state_item<D, PHI, false>(p, item);
        __syncthreads();  // the next item refills the ring
    }
    // then the step's overlap copy (these workgroups finish well before the
    // local launch they run beside)
    if (p.copy.keep_rows > 0) {
        const int cpr = p.copy.d * p.copy.elem_bytes / 16;
        const long long total = (long long)p.copy.BH * p.copy.keep_rows * cpr;
        const int nt = state_nw(D, PHI) * 64;
        for (long long idx = (long long)blockIdx.x * nt + threadIdx.x; idx < total; idx += (long long)gridDim.x * nt)
            prev_copy_chunk(p.copy, cpr, idx);
    }
}

template <int D>
hipError_t launch_d(const StateParams& p, hipStream_t s) {
    const long long items = (long long)p.BH * p.items_per_bh;
    if (items <= 0) return hipSuccess;
    const long long blocks = p.wg_items > 1 ? (items + p.wg_items - 1) / p.wg_items : items;
    switch (p.phi) {
    case kPhiElu1:
        if (p.row_lse) state_bf16_kernel<D, kPhiElu1, true><<<(unsigned)blocks, state_nw(D, kPhiElu1) * 64, 0, s>>>(p);
        else if (p.wg_items > 1) state_bf16_multi_kernel<D, kPhiElu1><<<(unsigned)blocks, state_nw(D, kPhiElu1) * 64, 0, s>>>(p);
        else state_bf16_kernel<D, kPhiElu1><<<(unsigned)blocks, state_nw(D, kPhiElu1) * 64, 0, s>>>(p);
        break;
    case kPhiPoly2:
        if (p.row_lse) state_bf16_kernel<D, kPhiPoly2, true><<<(unsigned)blocks, state_nw(D, kPhiPoly2) * 64, 0, s>>>(p);
        else if (p.wg_items > 1) state_bf16_multi_kernel<D, kPhiPoly2><<<(unsigned)blocks, state_nw(D, kPhiPoly2) * 64, 0, s>>>(p);
        else state_bf16_kernel<D, kPhiPoly2><<<(unsigned)blocks, state_nw(D, kPhiPoly2) * 64, 0, s>>>(p);
        break;
    case kPhiFeat: state_bf16_kernel<D, kPhiFeat><<<(unsigned)blocks, state_nw(D, kPhiFeat) * 64, 0, s>>>(p); break;
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
