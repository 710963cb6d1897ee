// proj.hip -- the projections of the attention block around the hybrid
// attention, bf16 MFMA GEMMs with fused epilogues.
//
// ReHyAt (arXiv 2601.04342) replaces the attention A_l of a DiT block
// T_l(x) = f_l(A_l(x) + x) (§3.1, first display equation) in 15, 20 or 25 of
// the 30 blocks of Wan2.1 1.3B (§4.3 "Model Hyperparameters").  Around the
// attention sit its input and output projections:
//   q = x Wq^T + bq,  k = (x Wk^T + bk) / sqrt(d),  v = x Wv^T + bv   (split into heads)
//   A(x) = concat_heads(attn(q, k, v)) Wo^T + bo,   block output x + A(x).
// The 1/sqrt(d) softmax scale is folded into k, the convention of the
// attention entry points.  Weights use the out x in layout of a linear layer.
//
// One kernel, two epilogues.  A workgroup of 4 waves forms a 128-feature x
// 128-token tile of the transposed product C^T = W X^T on
// v_mfma_f32_32x32x16_bf16 (A = W rows, B = X rows: both operands are rows
// with the reduction dimension contiguous, so every fragment is one 16-byte
// LDS read).  The large tiles: 256 features x 256 tokens, 8 waves of 128 x 64
// (4 x 2 MFMA tiles), W and X tiles of 64 input features double-buffered in
// LDS; the small ones (any width that is a multiple of 128): 128 x 128, 4 waves
// of 64 x 64, tiles of 32 input features in a 4-stage ring.  Tiles arrive by
// direct global->LDS loads, rows XOR-swizzled.  In the C
// layout a lane holds one token and, per group of four registers, four
// consecutive features, so the epilogue stores 8 bytes at a time:
//   QKV: + bias, k scaled by 1/sqrt(d), bf16, scattered to q, k, v in the
//        [B][H][N][d] layout the attention takes;
//   OUT: X rows are gathered from the attention output's [B][H][N][d] layout
//        (a k-tile lies within one head), + bias + the residual x,
//        bf16, token-major [B*N][C].
#include "local_common.h"

namespace rehyat {

namespace {

constexpr int kProjMinBK = 32;  // input features per LDS stage, at least
constexpr int kProjMinBF = 128;

// Tile configurations: workgroup tile BF features x BT tokens, NW waves in a
// WGF x (NW / WGF) grid, each wave (BF / WGF) features x (BT * WGF / NW)
// tokens, NS LDS stages of BK input features.  Measured at the Wan shape (QKV
// projection, one process): 256 x 256 with 3 stages of 32 features 550 us,
// with 4 stages 551 us, with 2 stages of 64 features 513 us; 4 waves of 128 x
// 128 (accumulators in AGPRs, one wave per SIMD) 679 us.
struct ProjCfg {
    int BF, BT, NW, WGF, NS, BK;
};
constexpr ProjCfg kProjCfgs[3] = {{128, 128, 4, 2, 4, 32}, {256, 256, 8, 2, 2, 64}, {256, 128, 8, 4, 4, 32}};
#ifndef REHYAT_PROJ_CFG
#define REHYAT_PROJ_CFG 1
#endif

// The body, instantiated per (epilogue, configuration) and wrapped by one
// kernel per configuration below (with the configuration as a second template
// parameter of the kernel itself, its host stubs were not emitted).
template <int MODE, int CFG>
__device__ __forceinline__ void proj_body(const ProjParams& p) {
    constexpr int BF = kProjCfgs[CFG].BF, BT = kProjCfgs[CFG].BT, NW = kProjCfgs[CFG].NW;
    constexpr int WGF = kProjCfgs[CFG].WGF, NS = kProjCfgs[CFG].NS;
    constexpr int BK = kProjCfgs[CFG].BK;
    constexpr int WGT = NW / WGF;
    constexpr int MI = BF / WGF / 32, NJ = BT / WGT / 32;  // 32x32 MFMA tiles per wave
    constexpr int CK = BK / 8;                       // 16-byte chunks per tile row
    constexpr int WT = BF * BK, XT = BT * BK;        // elements per W / X tile
    constexpr int STAGE = WT + XT;
    constexpr int NIW = WT * 2 / 1024, NIX = XT * 2 / 1024;  // 1 KB load instructions
    constexpr int OPW = (NIW + NIX) / NW;
    static_assert((NIW + NIX) % NW == 0 && NIW % NW == 0, "loads must split evenly over the waves");

    __shared__ __attribute__((aligned(16))) uint16_t smem_raw[NS * STAGE];
    lds_u16* const smem = (lds_u16*)smem_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5;
    const int lq = lane & 31;
    const int wf = wave / WGT, wt = wave % WGT;      // the wave's 32 MI features x 32 NJ tokens

    // tile order: feature tiles fastest, so the workgroups on an XCD share X rows
    const int nft = p.n_out / BF;
    const int item = xcd_remap(blockIdx.x, gridDim.x);
    const int f0 = (item % nft) * BF;
    const int t0 = (item / nft) * BT;
    const int C = p.c_in;

    const uint16_t* wb = (const uint16_t*)p.w + (long long)f0 * C;
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc((void*)wb, (short)0, BF * C * 2, 0x00020000);
    __amdgpu_buffer_rsrc_t xrs;
    const int t_rows = min(BT, p.T - t0);
    if constexpr (MODE == kProjQKV) {
        const uint16_t* xb = (const uint16_t*)p.x + (long long)t0 * C;
        xrs = __builtin_amdgcn_make_buffer_rsrc((void*)xb, (short)0, t_rows * C * 2, 0x00020000);
    } else {
        xrs = __builtin_amdgcn_make_buffer_rsrc((void*)p.x, (short)0, p.x_bytes, 0x00020000);
    }

    // per load op: tile row and the byte offset of its logical chunk within the row
    int op_row[OPW], op_c16[OPW];
    bool op_x[OPW];
#pragma unroll
    for (int o = 0; o < OPW; ++o) {
        const int op = wave + o * NW;
        op_x[o] = op >= NIW;
        const int ins = op_x[o] ? op - NIW : op;
        const int pos = 64 * ins + lane;
        op_row[o] = pos / CK;
        op_c16[o] = ((pos % CK) ^ swz<CK>(pos / CK)) * 16;
    }
    // OUT: token row -> element offset of its (b, n) row in head 0 of the
    // [B][H][N][d] attention output (tokens past T read beyond the tensor: zero)
    int xrow_base[OPW];
#pragma unroll
    for (int o = 0; o < OPW; ++o) {
        if constexpr (MODE == kProjOut) {
            const int t = t0 + op_row[o];
            const int b = t / p.N, n = t - (t / p.N) * p.N;
            xrow_base[o] = t < p.T ? (b * p.H * p.N + n) * p.d : p.x_bytes / 2;
        } else {
            xrow_base[o] = 0;
        }
    }
    auto issue = [&](int kt, lds_u16* st) {
        const int k0 = kt * BK;
#pragma unroll
        for (int o = 0; o < OPW; ++o) {
            const int op = wave + o * NW;
            const int ins = op_x[o] ? op - NIW : op;
            auto* lds = (__attribute__((address_space(3))) void*)(st + (op_x[o] ? WT : 0) + 512 * ins);
            if (!op_x[o]) {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, lds, 16, op_row[o] * C * 2 + k0 * 2 + op_c16[o], 0, 0, 0);
            } else if constexpr (MODE == kProjQKV) {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, lds, 16, op_row[o] * C * 2 + k0 * 2 + op_c16[o], 0, 0, 0);
            } else {
                const int hh = k0 / p.d, dd0 = k0 - (k0 / p.d) * p.d;
                const int off = (xrow_base[o] + hh * p.N * p.d + dd0) * 2 + op_c16[o];
                __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, lds, 16, xrow_base[o] * 2 >= p.x_bytes ? p.x_bytes : off,
                                                         0, 0, 0);
            }
        }
    };

    f32x16 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{};

    const int nk = C / BK;
    for (int kt = 0; kt < NS - 1 && kt < nk; ++kt) issue(kt, smem + kt * STAGE);
    for (int kt = 0; kt < nk; ++kt) {
        const int ahead = min(NS - 2, nk - 1 - kt);
        if (ahead >= 2) __builtin_amdgcn_s_waitcnt(vm_wait_imm(2 * OPW));
        else if (ahead == 1) __builtin_amdgcn_s_waitcnt(vm_wait_imm(OPW));
        else __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
        lds_barrier();
        if (kt + NS - 1 < nk) issue(kt + NS - 1, smem + ((kt + NS - 1) % NS) * STAGE);
        const lds_u16* Ws = smem + (kt % NS) * STAGE;
        const lds_u16* Xs = Ws + WT;
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            bf16x8 a[MI], b[NJ];
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const int rw = 32 * (MI * wf + i) + lq;
                a[i] = lds_read_b128(Ws, rw * BK + (((2 * s + h) ^ swz<CK>(rw)) << 3));
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int rx = 32 * (NJ * wt + j) + lq;
                b[j] = lds_read_b128(Xs, rx * BK + (((2 * s + h) ^ swz<CK>(rx)) << 3));
            }
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j) acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j]);
        }
    }

    // ---- epilogue: lane holds token t0 + 32 (NJ wt + j) + lq; register 4g + e is
    // feature f0 + 32 (MI wf + i) + 8 g + 4 h + e
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int t = t0 + 32 * (NJ * wt + j) + lq;
        if (t >= p.T) continue;
        const int b = t / p.N, n = t - (t / p.N) * p.N;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int f = f0 + 32 * (MI * wf + i) + 8 * g + 4 * h;
                const f32x4 bias = *(const f32x4*)(p.bias + f);
                float y[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = acc[i][j][4 * g + e] + bias[e];
                if constexpr (MODE == kProjQKV) {
                    const int which = f / C, within = f - which * C;
                    const int hh = within / p.d, dd = within - hh * p.d;
                    if (which == 1) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) y[e] *= p.k_scale;
                    }
                    uint16_t* dst = (uint16_t*)(which == 0 ? p.q : (which == 1 ? p.k : p.v));
                    const u32x2 w = {pack2_bf16(y[0], y[1]), pack2_bf16(y[2], y[3])};
                    *(u32x2*)(dst + ((long long)(b * p.H + hh) * p.N + n) * p.d + dd) = w;
                } else {
                    const u32x2 r = *(const u32x2*)((const uint16_t*)p.resid + (long long)t * p.n_out + f);
                    const float rr[4] = {__uint_as_float(r[0] << 16), __uint_as_float(r[0] & 0xffff0000u),
                                         __uint_as_float(r[1] << 16), __uint_as_float(r[1] & 0xffff0000u)};
                    const u32x2 w = {pack2_bf16(y[0] + rr[0], y[1] + rr[1]), pack2_bf16(y[2] + rr[2], y[3] + rr[3])};
                    *(u32x2*)((uint16_t*)p.out + (long long)t * p.n_out + f) = w;
                }
            }
    }
}

template <int MODE>
__global__ __launch_bounds__(64 * 4) void proj_bf16_small_kernel(ProjParams p) {
    proj_body<MODE, 0>(p);
}
template <int MODE>
__global__ __launch_bounds__(64 * 8) void proj_bf16_kernel(ProjParams p) {
    proj_body<MODE, REHYAT_PROJ_CFG>(p);
}

}  // namespace

bool proj_shape_ok(int c_in, int n_out, int head_dim) {
    return c_in % kProjMinBK == 0 && n_out % kProjMinBF == 0 && head_dim % kProjMinBK == 0 && c_in % head_dim == 0;
}

hipError_t launch_proj_bf16(const ProjParams& p, hipStream_t s) {
    // the larger tiles where the features and the input width split into them
    // (OUT gathers its input by heads: a k-tile must lie within one head), else
    // 128 x 128
    const ProjCfg c = kProjCfgs[REHYAT_PROJ_CFG];
    const bool big = REHYAT_PROJ_CFG != 0 && p.n_out % c.BF == 0 && p.c_in % c.BK == 0 && p.d % c.BK == 0;
    const ProjCfg u = big ? c : kProjCfgs[0];
    const long long tiles = (long long)(p.n_out / u.BF) * ((p.T + u.BT - 1) / u.BT);
    if (tiles <= 0) return hipSuccess;
    if (big) {
        if (p.mode == kProjQKV) proj_bf16_kernel<kProjQKV><<<(unsigned)tiles, u.NW * 64, 0, s>>>(p);
        else proj_bf16_kernel<kProjOut><<<(unsigned)tiles, u.NW * 64, 0, s>>>(p);
    } else {
        if (p.mode == kProjQKV) proj_bf16_small_kernel<kProjQKV><<<(unsigned)tiles, u.NW * 64, 0, s>>>(p);
        else proj_bf16_small_kernel<kProjOut><<<(unsigned)tiles, u.NW * 64, 0, s>>>(p);
    }
    return hipGetLastError();
}

}  // namespace rehyat
