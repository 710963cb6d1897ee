// kernels.h -- host-side launch interface between the C ABI (api.cpp) and the
// HIP kernels.  Plain structs of pointers and sizes; no torch types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rehyat {

// kPhiFeat: phi(q) and phi(k) come precomputed in feature buffers of D' = 2d
// columns (the learned map, see MlpParams) instead of being applied to q and k.
enum Phi { kPhiNone = 0, kPhiElu1 = 1, kPhiPoly2 = 2, kPhiFeat = 3 };

inline int feature_dim(int phi, int d) {
    return phi == kPhiElu1 ? d : ((phi == kPhiPoly2 || phi == kPhiFeat) ? 2 * d : 0);
}

// Partition of the keys into the blocks whose linear sums the state pass forms
// (frame ranges, times tokens_per_frame for rows).
//  kCausal: the delta blocks E_u = frames [max(u T_c - T_o, 0), max((u+1) T_c - T_o, 0)),
//   u = 0 .. C-2: the keys that leave the softmax window between chunk u and
//   u+1, so the linear set of chunk t (ReHyAt §3.3) is E_0 + ... + E_{t-1}.
//  kBidirectional: the frames cut at every c T_c - r and c T_c (r = T_o mod
//   T_c), clipped to [0, F): block 2c = [c T_c - r, c T_c), block 2c+1 =
//   [c T_c, (c+1) T_c - r), c = 0 .. C (2C+1 blocks).  The softmax window of
//   chunk t (§3.2, with overlap) starts at the start of block 2(t - q), q =
//   T_o div T_c (clipped at block 0), and ends at the start of block 2t+3, so
//   its linear set (every key outside the window) is the blocks before
//   max(2(t - q), 0) plus the blocks from 2t+3 on.
//  kChunkRows (backward): block u = the frames of chunk u+1, u = 0 .. C-2
//   (the queries whose gradient sums feed the keys of the earlier delta blocks).
//  kChunkRowsAll (backward of the bidirectional form): block u = chunk u.
//  kBidirGrad (scan only): slot b = sum over the chunks whose linear set holds
//   the bidirectional block b (see scan.hip).
enum BlockMode { kCausal = 0, kBidirectional = 1, kChunkRows = 2, kChunkRowsAll = 3, kBidirGrad = 4 };

__host__ __device__ inline int state_block_count(int mode, int C) {
    return mode == kBidirectional ? 2 * C + 1 : (mode == kChunkRowsAll ? C : C - 1);
}

// Bidirectional block of frame f: block 2c = [c T_c - r, c T_c), 2c+1 = [c T_c, (c+1) T_c - r).
__host__ __device__ inline int bidir_block_of_frame(int f, int Tc, int To) {
    const int r = To % Tc;
    const int c = (f + r) / Tc;
    return f < c * Tc ? 2 * c : 2 * c + 1;
}

__host__ __device__ inline void state_block_frames(int mode, int u, int Tc, int To, int F, int& f0, int& f1) {
    if (mode == kChunkRows || mode == kChunkRowsAll) {
        const int c = mode == kChunkRows ? u + 1 : u;
        f0 = c * Tc < F ? c * Tc : F;
        f1 = (c + 1) * Tc < F ? (c + 1) * Tc : F;
        return;
    }
    if (mode == kCausal) {
        f0 = u * Tc - To > 0 ? u * Tc - To : 0;
        f1 = (u + 1) * Tc - To > 0 ? (u + 1) * Tc - To : 0;
        return;
    }
    const int r = To % Tc, c = u >> 1;
    int a, b;
    if ((u & 1) == 0) {
        a = c * Tc - r;
        b = c * Tc;
    } else {
        a = c * Tc;
        b = (c + 1) * Tc - r;
    }
    f0 = a < 0 ? 0 : (a > F ? F : a);
    f1 = b < 0 ? 0 : (b > F ? F : b);
}

// Local-softmax + fused hybrid combine (one launch covers every (b, h, chunk,
// query tile)).  Key rows of a window are addressed through a virtual index j:
// j < prev_rows reads the "prev" segment (the streaming overlap frames), the
// rest read the clip from row w0 of the chunk's window.
struct LocalParams {
    const void* q;            // [BH][n_rows][d] queries (clip or chunk)
    void* out;                // same layout as q
    const void* k;            // [BH][n_rows][d]
    const void* v;
    const void* kp;           // [BH][prev_stride_rows][d] overlap segment (streaming), or null
    const void* vp;
    long long bh_stride;      // n_rows * d
    long long prev_bh_stride; // rows per (b,h) in kp/vp times d
    int prev_rows;            // rows of the overlap segment in front of the window
    int HW, F, Tc, To;        // frames / chunk geometry of this launch
    int n_chunks, tiles_per_chunk, BH;
    int d;
    // linear branch: prepared state for each (bh, chunk)
    int phi;                  // Phi
    int lin_always;           // linear branch active for every chunk (streaming, state nonempty)
    const void* s_hi;         // bf16 [d][D'] hi part of S^T  (fp32 path: fp32 S^T here, s_lo unused)
    const void* s_lo;         // bf16 [d][D'] lo part
    const float* z;           // fp32 [D']
    long long s_chunk_stride; // elements between consecutive chunks' prepared states
    long long s_bh_stride;    // elements between consecutive (b,h)
    long long z_chunk_stride, z_bh_stride;
    // optional partials (verification aid): fp32
    float* pm; float* pnt; float* poS; float* poL; float* pnL;
    int lpt_order;            // dispatch each XCD's work items longest first (see local_work_item)
    // kPhiFeat: phi(q) rows, [BH][n_rows][2d] in the input dtype (row = query row)
    const void* fq;
    long long fq_bh_stride;
    // optional: ln(n^S + n^L) per query, fp32 [BH][n_rows] (the backward's normaliser)
    float* lse;
    // optional (bf16 path): the output before rounding, fp32, same layout as out
    float* out_f32;
};

// Key tiles of BN keys that a query tile of chunk t streams (its softmax window).
__host__ __device__ inline int chunk_key_tiles(const LocalParams& p, int t, int BN) {
    const int f0 = t * p.Tc;
    const int f1 = f0 + p.Tc < p.F ? f0 + p.Tc : p.F;
    const int w0 = f0 - p.To > 0 ? f0 - p.To : 0;
    const int nkeys = p.prev_rows + (f1 - w0) * p.HW;
    return (nkeys + BN - 1) / BN;
}

// Work item of workgroup `bid` of the local kernel.  The dispatcher deals
// workgroups round-robin over the 8 XCDs, so workgroup bid is the (bid / 8)-th
// one XCD bid % 8 receives, and each XCD hands its workgroups to its CUs as
// they free up.  Each XCD owns a contiguous share of the items (item = (bh *
// n_chunks + t) * tiles_per_chunk + query tile), so the query tiles of a chunk
// share that XCD's L2.  With lpt_order the share is taken in order of
// decreasing cost (key tiles of the chunk), chunk by chunk, so the greedy
// assignment ends on the short items; otherwise in natural order.
__host__ __device__ inline int local_work_item(const LocalParams& p, int bid, int nblocks, int BN) {
    const int per = nblocks / 8, tail = nblocks % 8;
    const int xcd = bid % 8, idx = bid / 8;
    const int s = xcd < tail ? xcd * (per + 1) : tail * (per + 1) + (xcd - tail) * per;
    if (!p.lpt_order) return s + idx;
    const int e = s + per + (xcd < tail ? 1 : 0);
    const int T = p.tiles_per_chunk;
    const int gs = s / T, ge = (e - 1) / T;  // chunk groups meeting [s, e)
    int rem = idx, level = 1 << 30;
    for (;;) {
        int c = -1;  // the largest cost below `level`
        for (int g = gs; g <= ge; ++g) {
            const int cg = chunk_key_tiles(p, g % p.n_chunks, BN);
            if (cg < level && cg > c) c = cg;
        }
        if (c < 0) return s + idx;  // unreachable: every position lies in some group
        for (int g = gs; g <= ge; ++g) {
            if (chunk_key_tiles(p, g % p.n_chunks, BN) != c) continue;
            const int a = g * T > s ? g * T : s;
            const int b = (g + 1) * T < e ? (g + 1) * T : e;
            if (rem < b - a) return a + rem;
            rem -= b - a;
        }
        level = c;
    }
}

// Copy of the last `keep_rows` rows of [prev | chunk] into the other overlap slot
// (K, V and, for the learned map, phi(K) rows of f_cols columns).
struct PrevCopyParams {
    const void* kp; const void* vp; long long prev_bh_stride; int prev_rows;
    const void* k; const void* v; long long bh_stride; int chunk_rows;
    void* kd; void* vd;               // destination slot, same stride as prev
    int keep_rows, BH, d, elem_bytes;
    const void* fkp; const void* fk; void* fkd;   // phi(K) rows or null
    long long fprev_bh_stride, f_bh_stride;
    int f_cols;
};

// Block-state pass: partial S^T = sum phi(k) v^T (stored [d][D'] fp32) and
// z = sum phi(k) over contiguous key sub-blocks of each delta block E_u.
struct StateParams {
    const void* k; const void* v;     // [BH][n_rows][d]
    const void* kp; const void* vp;   // overlap segment (streaming) or null
    long long bh_stride, prev_bh_stride;
    int prev_rows;
    int HW, Tc, To;                   // delta block u covers frames [max(uTc-To,0), max((u+1)Tc-To,0))
    int n_blocks;                     // U: number of delta blocks
    int sub_rows;                     // key rows per sub-block
    int n_sub;                        // sub-blocks per delta block (max over blocks): the partial stride
    int items_per_bh;                 // workgroups per (b, h): the sub-blocks of all blocks
    int stream_rows;                  // streaming: rows of [prev | chunk] to fold (U = 1); 0 in fwd
    int BH, d, phi;
    int mode, F;                      // block partition (BlockMode) and frames of the clip
    float* partial;                   // [BH][U][n_sub][d*D' + D']
    // kPhiFeat: phi(k) rows in the input dtype, [BH][n_rows][2d] and for the
    // overlap segment [BH][prev rows][2d] (indexed like k and kp)
    const void* fk; const void* fkp;
    long long fk_bh_stride, fkp_bh_stride;
    // backward (kChunkRows): row r contributes c_r phi(x_r) v_r^T to S and
    // D_r c_r phi(x_r) to z, c_r = exp(-row_lse[r]), D_r = row_d[r] ([BH][n_rows])
    const float* row_lse; const float* row_d;
    // bf16 elu+1 / poly2: sub-blocks per workgroup (0 or 1: one workgroup each);
    // more: fewer workgroups take the sub-blocks in turn (same results)
    int wg_items;
    // with wg_items > 1 (the streaming fold): the overlap copy of the step,
    // done by the same workgroups after their sub-blocks (keep_rows 0: none)
    PrevCopyParams copy;
};

// The blocks of a state partition and their sub-blocks: block u covers rows
// [e0, e1) (a single block of stream_rows rows in a streaming fold) and is
// split into sub-blocks of sub_rows rows, one workgroup and one partial sum
// each; an empty block has none (its sum is zero).
struct BlockPart {
    int mode, HW, Tc, To, F, stream_rows, sub_rows;
};

__host__ __device__ inline BlockPart state_part(const StateParams& p) {
    return BlockPart{p.mode, p.HW, p.Tc, p.To, p.F, p.stream_rows, p.sub_rows};
}

__host__ __device__ inline void part_block_rows(const BlockPart& b, int u, int& e0, int& e1) {
    if (b.stream_rows > 0) {
        e0 = 0;
        e1 = b.stream_rows;
        return;
    }
    int fa, fb;
    state_block_frames(b.mode, u, b.Tc, b.To, b.F, fa, fb);
    e0 = fa * b.HW;
    e1 = fb * b.HW;
}

__host__ __device__ inline int part_block_subs(const BlockPart& b, int u) {
    int e0, e1;
    part_block_rows(b, u, e0, e1);
    return e1 > e0 ? (e1 - e0 + b.sub_rows - 1) / b.sub_rows : 0;
}

// Scan: X_0 = init (or 0); X_{u+1} = X_u + sum_p partial[u][p].  Writes the
// prepared form of X_t for t in [t_first, U] and, if state_out, X_U in fp32.
struct ScanParams {
    const float* partial;             // [BH][U][n_sub][E], block u in its first part_block_subs(u) slots
    BlockPart part;                   // the blocks the partial sums were made over
    const float* init;                // [BH][E] or null
    float* state_out;                 // [BH][E] or null (may alias init)
    void* s_hi; void* s_lo;           // prepared S^T per (bh, t) (bf16 hi/lo, or fp32 in s_hi)
    float* z;                         // prepared z per (bh, t)
    long long s_chunk_stride, s_bh_stride, z_chunk_stride, z_bh_stride;
    int U, n_sub, BH, d, Dp;
    int t_first;                      // first prepared state to write
    int t_offset;                     // prepared state X_t is written at slot t - t_offset
    int f32_prep;                     // prepared form is fp32 (s_hi) rather than bf16 hi/lo
    // kBidirectional: U = 2C+1 blocks; chunk t gets the sum of the blocks
    // before max(2(t - q), 0) plus the blocks from 2t+3 on (q = T_o div T_c)
    int mode, C, q;
    float* suffix;                    // [BH][C][E] fp32 scratch for the suffix sums
    // kChunkRows (backward): slot u gets the sum of the blocks u .. U-1
    // optional copy of each prepared S^T transposed, [D'][d] (bf16 hi/lo, or fp32 in t_hi)
    void* t_hi; void* t_lo;
};

// Backward of the hybrid attention (per-chunk windows of the recurrent form).
// dq, dk, dv in the input dtype.  lse = ln(n^S + n^L) and dsum = dy.y per query.
struct BwdParams {
    const void* q; const void* k; const void* v; const void* dy;  // [BH][N][d]
    const void* out;                                              // forward output (for dsum)
    const float* out_f32;                                         // or its fp32 copy (bf16 path), preferred
    const float* lse; const float* dsum;                          // [BH][N]
    void* dq; void* dk; void* dv;
    long long bh_stride;                                          // N * d
    int N, HW, F, Tc, To, C, BH, d, phi;
    // linear branch, per chunk t: the forward state S_t prepared transposed
    // ([D'][d], bf16 hi/lo or fp32) and z_t; per delta block u: the suffix of
    // the gradient sums, G_u = sum_{t>u} sum_{i in chunk t} e^{-lse_i} phi(q_i) dy_i^T,
    // prepared as G_u^T [d][D'] and G_u [D'][d], and g_u = sum e^{-lse_i} dsum_i phi(q_i)
    const void* st_hi; const void* st_lo; const float* z;
    const void* g_hi; const void* g_lo; const void* gt_hi; const void* gt_lo; const float* gz;
    long long s_stride, z_stride;     // per chunk / per block: d*D' and D' elements (bh stride = C times)
    int lin;                          // the linear branch is active (some chunk has a linear set)
    int mode;                         // kCausal or kBidirectional (then: G per bidirectional block,
                                      // 2C+1 slots, and every chunk has a linear set)
    int dq_lpt;                       // dq workgroups: each XCD's items longest first (local_work_item)
};

// Learned feature map (ReHyAt §3.2 polynomial form with a two-layer MLP, §4.3 /
// appendix §7.1): for every row x of the selected rows,
//   psi = W2 relu(W1 x + b1) + b2   (2d values),  phi(x) = [1 + elu(psi[0:d]), psi[d:2d]^2],
// per head, with separate weights for queries and keys (one "side" each).
struct MlpSide {
    const void* x;                    // [BH][.][d] rows in the input dtype
    void* out;                        // [BH][.][2d] phi rows, input dtype; row r of x -> row r of out
    const void* w1;                   // [H][hidden][d], input dtype
    const float* b1;                  // [H][hidden]
    const void* w2;                   // [H][2d][hidden], input dtype
    const float* b2;                  // [H][2d]
    long long x_bh_stride, out_bh_stride;  // elements between consecutive (b, h)
    int r0, r1;                       // rows [r0, r1) of every (b, h) are mapped
};
struct MlpParams {
    MlpSide side[2];
    int n_sides, BH, H, d, hidden;
    int grid;                         // workgroups (bf16 kernel: at most one per CU)
};

// Projections of the attention block (bf16 MFMA GEMM, C^T = W X^T per tile):
//  kProjQKV: x [T][C] token-major, w [3C][C] (out x in), bias [3C] ->
//            q, k, v [B][H][N][d] (k times k_scale)
//  kProjOut: x = the attention output [B][H][N][d], w [C][C], bias [C], resid
//            [T][C] -> out [T][C] = resid + x Wo^T + bias
enum ProjMode { kProjQKV = 0, kProjOut = 1 };
struct ProjParams {
    int mode;
    const void* x;                    // bf16, see above
    int x_bytes;                      // kProjOut: bytes of the attention output (reads past it give 0)
    const void* w;                    // bf16 [n_out][c_in]
    const float* bias;                // [n_out]
    void* q; void* k; void* v;        // kProjQKV outputs
    float k_scale;
    const void* resid; void* out;     // kProjOut
    int T, N, H, d, c_in, n_out;      // tokens (B*N), tokens per batch entry, heads, head_dim
};
bool proj_shape_ok(int c_in, int n_out, int head_dim);
hipError_t launch_proj_bf16(const ProjParams& p, hipStream_t s);

hipError_t launch_local_bf16(const LocalParams& p, hipStream_t s);
hipError_t launch_local_f32(const LocalParams& p, hipStream_t s);
hipError_t launch_state_bf16(const StateParams& p, hipStream_t s);
hipError_t launch_state_f32(const StateParams& p, hipStream_t s);
hipError_t launch_scan(const ScanParams& p, hipStream_t s);
hipError_t launch_prev_copy(const PrevCopyParams& p, hipStream_t s);
// scan and copy in one launch (either may be null)
hipError_t launch_scan_copy(const ScanParams* sp, const PrevCopyParams* pc, hipStream_t s);
hipError_t launch_phi_mlp_bf16(const MlpParams& p, hipStream_t s);
hipError_t launch_bwd_dsum(const BwdParams& p, float* dsum, bool bf16, hipStream_t s);  // dsum = rowwise dy . out
hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t s);   // dq, dk, dv
// The bf16 dq kernel's work items: query tiles per chunk and keys per tile (for
// the host's choice of dispatch order).
void dq_launch_shape(const BwdParams& p, int& tiles_per_chunk, int& key_tile);
hipError_t launch_bwd_f32(const BwdParams& p, hipStream_t s);
hipError_t launch_phi_mlp_f32(const MlpParams& p, hipStream_t s);
bool phi_mlp_hidden_ok(int hidden);  // hidden widths the MLP kernels are built for

int local_bf16_tile_rows(int d);   // queries per workgroup of the bf16 local kernel
int local_bf16_key_tile(int d);    // keys per LDS tile of the bf16 local kernel
int local_f32_tile_rows(int d);

}  // namespace rehyat
