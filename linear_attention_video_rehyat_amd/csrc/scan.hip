// scan.hip -- cross-chunk carry of the linear state and the overlap-frame copy.
//
// The chunk-wise RNN form of ReHyAt (arXiv 2601.04342, §3.3) carries the cached
// linear sums S = sum phi(k) v^T and z = sum phi(k) (§3.1) from chunk to chunk:
// chunk t sees X_t = sum_{u<t} E_u, the sums of every delta block that left the
// softmax window before it.  This kernel forms that exclusive prefix in fp32,
// sequentially in u (one thread per 4 state elements), and writes each X_t in
// the form the local kernel's epilogue consumes: S^T split into bf16 hi + lo
// parts (or fp32 for the fp32 path) and z in fp32.  For the bidirectional form
// (§3.2 with overlap: the linear set is every key outside the window, later
// chunks included) the state of chunk t is a prefix plus a suffix of the block
// sums, kept as two separate sums rather than a total minus the window.
#include "common.h"
#include "copy_rows.h"
#include "kernels.h"

namespace rehyat {

namespace {

// Elements e4 .. e4+3 of the state of (b, h) bh.
__device__ __forceinline__ void scan_elem(const ScanParams& p, const int bh, const int e4) {
    const int E = p.d * p.Dp + p.Dp;
    const long long pstride = (long long)E;  // between sub-blocks
    const float* part = p.partial + (long long)bh * p.U * p.n_sub * E + e4;
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (p.init) x = *(const f32x4*)(p.init + (long long)bh * E + e4);
    const int SE = p.d * p.Dp;
    auto emit = [&](int t) {
        if (t < p.t_first) return;
        const int slot = t - p.t_offset;
        if (e4 < SE) {
            const long long base = (long long)bh * p.s_bh_stride + (long long)slot * p.s_chunk_stride;
            const long long off = base + e4;
            if (p.f32_prep) {
                *(f32x4*)((float*)p.s_hi + off) = x;
            } else {
                uint32_t hi[2], lo[2];
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const u32x2 hl = split2_bf16(x[2 * j], x[2 * j + 1]);
                    hi[j] = hl[0];
                    lo[j] = hl[1];
                }
                *(u32x2*)((uint16_t*)p.s_hi + off) = u32x2{hi[0], hi[1]};
                *(u32x2*)((uint16_t*)p.s_lo + off) = u32x2{lo[0], lo[1]};
            }
            if (p.t_hi) {  // the transposed copy: element (r, c) of [d][D'] goes to (c, r) of [D'][d]
                const int r = e4 / p.Dp, c = e4 - r * p.Dp;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const long long to = base + (long long)(c + i) * p.d + r;
                    if (p.f32_prep) {
                        ((float*)p.t_hi)[to] = x[i];
                    } else {
                        const float hv = round_bf16(x[i]);
                        ((__bf16*)p.t_hi)[to] = (__bf16)hv;
                        ((__bf16*)p.t_lo)[to] = (__bf16)(x[i] - hv);
                    }
                }
            }
        } else {
            const long long off = (long long)bh * p.z_bh_stride + (long long)slot * p.z_chunk_stride + (e4 - SE);
            *(f32x4*)(p.z + off) = x;
        }
    };
    // the sub-blocks' loads of a block sum are issued together (up to 4)
    auto block_sum = [&](int u) {
        const int n = part_block_subs(p.part, u);
        f32x4 d[4];
#pragma unroll
        for (int sp = 0; sp < 4; ++sp)
            d[sp] = sp < n ? *(const f32x4*)(part + ((long long)u * p.n_sub + sp) * pstride) : f32x4{0.f, 0.f, 0.f, 0.f};
        f32x4 b = d[0] + d[1] + d[2] + d[3];
        for (int sp = 4; sp < n; ++sp) b += *(const f32x4*)(part + ((long long)u * p.n_sub + sp) * pstride);
        return b;
    };
    if (p.mode == kChunkRows) {
        // suffix sums: slot u gets the blocks u .. U-1
        for (int u = p.U - 1; u >= 0; --u) {
            x += block_sum(u);
            emit(u);
        }
        return;
    }
    if (p.mode == kBidirGrad) {
        // blocks = chunks 0 .. C-1 (U = C).  Bidirectional block b lies in the
        // linear set of chunk t iff b < 2(t - q) or b >= 2t + 3, i.e. for
        // t >= q + b/2 + 1 (suffix over chunks) and t <= (b - 3)/2 (prefix).
        // Suffix sums Y_t = sum_{t' >= t} into scratch (Y_C = 0), then slot b =
        // prefix + Y[min(q + b/2 + 1, C)] for b = 0 .. 2C.
        float* suf = p.suffix + (long long)bh * (p.C + 1) * E + e4;
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
        *(f32x4*)(suf + (long long)p.C * E) = y;
        for (int t = p.C - 1; t >= 0; --t) {
            y += block_sum(t);
            *(f32x4*)(suf + (long long)t * E) = y;
        }
        int pt = 0;  // chunks summed into the prefix x
        for (int b = 0; b <= 2 * p.C; ++b) {
            const int pe = b >= 3 ? (b - 3) / 2 + 1 : 0;  // prefix: chunks < pe
            for (; pt < min(pe, p.C); ++pt) x += block_sum(pt);
            const f32x4 keep = x;
            x += *(const f32x4*)(suf + (long long)min(p.q + b / 2 + 1, p.C) * E);
            emit(b);
            x = keep;
        }
        return;
    }
    if (p.mode == kBidirectional && p.U <= 16 && p.C <= 8 && p.n_sub <= 2) {
        // the same sums as below from block sums held in registers: every
        // load is issued at once (U <= 16 blocks of at most 2 sub-blocks)
        constexpr int MB = 16, MC = 8;
        f32x4 bs[MB];
#pragma unroll
        for (int k = 0; k < MB; ++k) {
            const int n = k < p.U ? part_block_subs(p.part, k) : 0;
            const f32x4 a = n > 0 ? *(const f32x4*)(part + ((long long)k * p.n_sub) * pstride) : f32x4{0.f, 0.f, 0.f, 0.f};
            const f32x4 b = n > 1 ? *(const f32x4*)(part + ((long long)k * p.n_sub + 1) * pstride) : f32x4{0.f, 0.f, 0.f, 0.f};
            bs[k] = a + b + f32x4{0.f, 0.f, 0.f, 0.f} + f32x4{0.f, 0.f, 0.f, 0.f};
        }
        // suffix Y_{2t+3} for every chunk (zero past the last block)
        f32x4 ys[MC];
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < MC; ++t) ys[t] = y;
#pragma unroll
        for (int k = MB - 1; k >= 0; --k) {
            if (k >= p.U) continue;
            y += bs[k];
#pragma unroll
            for (int t = 0; t < MC; ++t)
                if (k >= 3 && (k & 1) && (k - 3) / 2 == t && t < p.C) ys[t] = y;
        }
        // prefix sums, forwards; chunk t adds the blocks before max(2(t-q), 0)
        int k0 = 0;
#pragma unroll
        for (int t = 0; t < MC; ++t) {
            if (t >= p.C) break;
            const int pk = max(2 * (t - p.q), 0);
#pragma unroll
            for (int k = 0; k < MB; ++k)
                if (k >= k0 && k < pk) x += bs[k];
            k0 = max(k0, pk);
            const f32x4 keep = x;
            x += ys[t];
            emit(t);
            x = keep;
        }
        return;
    }
    if (p.mode == kBidirectional) {
        // suffix sums Y_k = sum of blocks k.. U-1, backwards; chunk t needs
        // Y_{2t+3} (zero past the last block).  Each thread keeps its own 4
        // elements, so the scratch needs no synchronisation.
        float* suf = p.suffix + (long long)bh * p.C * E + e4;
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
        for (int t = 0; t < p.C; ++t)
            if (2 * t + 3 >= p.U) *(f32x4*)(suf + (long long)t * E) = y;
        for (int k = p.U - 1; k >= 0; --k) {
            y += block_sum(k);
            if (k >= 3 && (k & 1) && (k - 3) / 2 < p.C) *(f32x4*)(suf + (long long)((k - 3) / 2) * E) = y;
        }
        // prefix sums, forwards; chunk t adds the blocks before max(2(t-q), 0)
        int k = 0;
        for (int t = 0; t < p.C; ++t) {
            const int pk = max(2 * (t - p.q), 0);
            for (; k < pk; ++k) x += block_sum(k);
            const f32x4 keep = x;
            x += *(const f32x4*)(suf + (long long)t * E);
            emit(t);
            x = keep;
        }
        return;
    }
    // The latency of the loads is what costs, not the short chain of adds:
    // up to 8 delta blocks of up to 4 sub-blocks, every load is issued at once
    constexpr int MAXU = 8, MAXS = 4;
    if (p.U <= MAXU && p.n_sub <= MAXS) {
        f32x4 d[MAXU][MAXS];
#pragma unroll
        for (int u = 0; u < MAXU; ++u) {
            const int n = u < p.U ? part_block_subs(p.part, u) : 0;
#pragma unroll
            for (int sp = 0; sp < MAXS; ++sp)
                d[u][sp] = sp < n ? *(const f32x4*)(part + ((long long)u * p.n_sub + sp) * pstride)
                                  : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < MAXU; ++u) {
            if (u >= p.U) break;
            emit(u);
            f32x4 b = d[u][0];
#pragma unroll
            for (int sp = 1; sp < MAXS; ++sp) b += d[u][sp];
            x += b;
        }
        emit(p.U);
        if (p.state_out) *(f32x4*)(p.state_out + (long long)bh * E + e4) = x;
        return;
    }
    // otherwise blocks of 4 delta blocks, their loads issued together
    for (int u0 = 0; u0 < p.U; u0 += 4) {
        f32x4 d[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            d[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (u0 + i < p.U) d[i] = block_sum(u0 + i);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (u0 + i >= p.U) break;
            emit(u0 + i);
            x += d[i];
        }
    }
    emit(p.U);
    if (p.state_out) *(f32x4*)(p.state_out + (long long)bh * E + e4) = x;
}

__global__ __launch_bounds__(256) void scan_kernel(ScanParams p) {
    const int e4 = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (e4 >= p.d * p.Dp + p.Dp) return;
    scan_elem(p, blockIdx.y, e4);
}

__global__ __launch_bounds__(256) void prev_copy_kernel(PrevCopyParams p) {
    const int cpr = p.d * p.elem_bytes / 16;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long long)p.BH * p.keep_rows * cpr) return;
    prev_copy_chunk(p, cpr, idx);
}

// A streaming step's update after its local launch, in one launch: the first
// scan_blocks workgroups add the fold into the state (as scan_kernel, the
// blocks of each (b, h) in turn), the others copy the kept rows.
__global__ __launch_bounds__(256) void scan_copy_kernel(ScanParams sp, PrevCopyParams pc, int scan_blocks) {
    if ((int)blockIdx.x < scan_blocks) {
        const int E = sp.d * sp.Dp + sp.Dp;
        const int bx = (E / 4 + 255) / 256;
        const int e4 = ((blockIdx.x % bx) * 256 + threadIdx.x) * 4;
        if (e4 < E) scan_elem(sp, blockIdx.x / bx, e4);
        return;
    }
    const int cpr = pc.d * pc.elem_bytes / 16;
    const long long idx = (long long)(blockIdx.x - scan_blocks) * 256 + threadIdx.x;
    if (idx < (long long)pc.BH * pc.keep_rows * cpr) prev_copy_chunk(pc, cpr, idx);
}

}  // namespace

hipError_t launch_scan(const ScanParams& p, hipStream_t s) {
    const int E = p.d * p.Dp + p.Dp;
    const int blocks = (E / 4 + 255) / 256;
    if (blocks <= 0 || p.BH <= 0) return hipSuccess;
    scan_kernel<<<dim3(blocks, p.BH), 256, 0, s>>>(p);
    return hipGetLastError();
}

namespace {
long long copy_chunks(const PrevCopyParams& p) { return (long long)p.BH * p.keep_rows * (p.d * p.elem_bytes / 16); }

void prev_copy_plane(const PrevCopyParams& p, hipStream_t s) {
    const long long total = copy_chunks(p);
    if (total > 0) prev_copy_kernel<<<dim3((unsigned)((total + 255) / 256)), 256, 0, s>>>(p);
}

// the phi(K) rows of the same frames, as a plane of their own
PrevCopyParams feature_plane(const PrevCopyParams& p) {
    PrevCopyParams f = p;
    f.kp = p.fkp; f.k = p.fk; f.kd = p.fkd;
    f.vp = nullptr; f.v = nullptr; f.vd = nullptr;
    f.prev_bh_stride = p.fprev_bh_stride; f.bh_stride = p.f_bh_stride; f.d = p.f_cols;
    return f;
}
}  // namespace

hipError_t launch_prev_copy(const PrevCopyParams& p, hipStream_t s) {
    prev_copy_plane(p, s);
    if (p.fkd) prev_copy_plane(feature_plane(p), s);
    return hipGetLastError();
}

hipError_t launch_scan_copy(const ScanParams* sp, const PrevCopyParams* pc, hipStream_t s) {
    if (!sp) return pc ? launch_prev_copy(*pc, s) : hipSuccess;
    if (!pc) return launch_scan(*sp, s);
    const int E = sp->d * sp->Dp + sp->Dp;
    const long long scan_blocks = (long long)((E / 4 + 255) / 256) * sp->BH;
    const long long copy_blocks = (copy_chunks(*pc) + 255) / 256;
    if (scan_blocks + copy_blocks > 0)
        scan_copy_kernel<<<dim3((unsigned)(scan_blocks + copy_blocks)), 256, 0, s>>>(*sp, *pc, (int)scan_blocks);
    if (pc->fkd) prev_copy_plane(feature_plane(*pc), s);
    return hipGetLastError();
}

}  // namespace rehyat
