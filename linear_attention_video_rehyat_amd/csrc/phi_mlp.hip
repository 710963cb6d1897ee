// phi_mlp.hip -- the learned feature map of ReHyAt as a fused two-layer MLP.
//
// ReHyAt (arXiv 2601.04342) writes phi as a concatenation of powers of learned
// functions psi_p (§3.2, the equation after the partitions) and makes them a
// two-layer MLP of degree 2, with separate maps for queries and keys (§4.3
// "Model Hyperparameters", appendix §7.1).  Per head and row x (d values):
//   hidden = relu(W1 x + b1)            (hidden values)
//   psi    = W2 hidden + b2             (2d values)
//   phi(x) = [1 + elu(psi[0:d]), psi[d:2d]^2]
// phi >= 0 everywhere, as §3.1 requires of a linear-attention feature map.
//
// bf16 kernel: both layers on MFMA (v_mfma_f32_32x32x16_bf16, fp32
// accumulation); the hidden layer and phi are rounded to bf16, the precision a
// bf16 model keeps its activations in.  A workgroup of 8 waves walks a
// contiguous run of 128-row blocks (queries, then keys, of every (b, h));
// each block of x lands in LDS by direct global->LDS loads (the next block's
// load is in flight during the current one), and every wave keeps its share of
// W1 and W2 in registers for as long as the head does not change:
//   layer 1: wave w forms hidden rows [32w, 32w+32) for the block's 128 rows,
//            H^T = W1 x^T (A = W1 from registers, B = x^T fragments from LDS),
//            and writes relu(. + b1) in bf16 to an LDS tile [128][hidden];
//   layer 2: wave w forms psi rows [32w, 32w+32) (one 32-wide feature tile),
//            psi^T = W2 H^T (A = W2 from registers, B = H^T fragments from LDS),
//            applies phi and stores its 32 columns of the 128 phi rows.
// fp32 kernel: the same map on the vector ALU in fp32.
#include <algorithm>

#include <type_traits>

#include "local_common.h"

namespace rehyat {

// Workgroup barrier after LDS writes that other waves read next: the barrier
// alone does not wait for the writing wave's LDS operations, so they are
// waited for first (s_waitcnt with lgkmcnt 0, vmcnt and expcnt at their maxima).
__device__ __forceinline__ void lds_write_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    lds_barrier();
}

namespace {

constexpr int kMlpRows = 128;  // rows per block
constexpr int kMlpWaves = 8;

__device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

// XOR swizzle of the 16-byte chunks of row r of the hidden tile (CH chunks per
// row): 16 consecutive rows read at one logical chunk hit 16 different
// 4-bank groups.
template <int CH>
__device__ __forceinline__ int hswz(int r) {
    return r & ((CH < 16 ? CH : 16) - 1);
}

// Block b of the walk -> (side, bh, first row relative to the side's r0).
__device__ __forceinline__ void mlp_block(const MlpParams& p, int nb0, int nb1, int b, int& side, int& bh,
                                          int& row0) {
    const int n0 = p.BH * nb0;
    side = b < n0 ? 0 : 1;
    const int rem = side ? b - n0 : b;
    const int nb = side ? nb1 : nb0;
    bh = rem / nb;
    row0 = (rem - bh * nb) * kMlpRows;
}

template <int D, int HID>
__global__ __launch_bounds__(kMlpRows * 4) void phi_mlp_bf16_kernel(MlpParams p) {
    constexpr int RB = kMlpRows, NW = kMlpWaves;
    constexpr int C = D / 8;                // 16-byte chunks per x row
    constexpr int CH = HID / 8;             // per hidden row
    constexpr int KS1 = D / 16, KS2 = HID / 16;
    constexpr int HT = HID / 32;            // hidden tiles (layer-1 waves)
    constexpr int FT = D / 16;              // 32-wide tiles of the 2d features (layer-2 waves)
    constexpr int XT = RB * D;              // elements of an x block
    constexpr int NI = XT * 2 / 1024;       // 1 KB loads per x block
    constexpr int OPW = NI / NW;
    static_assert(NI % NW == 0, "x block loads must split evenly over the waves");
    static_assert(HT <= NW && FT <= NW, "one tile per wave and layer");
    __shared__ __attribute__((aligned(16))) uint16_t xs_raw[2 * XT];
    __shared__ __attribute__((aligned(16))) uint16_t hs_raw[RB * HID];
    lds_u16* const xs = (lds_u16*)xs_raw;
    lds_u16* const hs = (lds_u16*)hs_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5;
    const int lq = lane & 31;

    const int nb0 = p.n_sides > 0 ? cdiv(max(p.side[0].r1 - p.side[0].r0, 0), RB) : 0;
    const int nb1 = p.n_sides > 1 ? cdiv(max(p.side[1].r1 - p.side[1].r0, 0), RB) : 0;
    const long long total = (long long)p.BH * (nb0 + nb1);
    const int g = xcd_remap(blockIdx.x, gridDim.x);
    const int b_begin = (int)(total * g / gridDim.x);
    const int b_end = (int)(total * (g + 1) / gridDim.x);
    if (b_begin >= b_end) return;

    // one wave's share of an x block (swizzled rows): loaded into registers
    // (xr) and written to the LDS slot later.  The per-lane byte offsets within
    // a block are fixed; the block's first row goes in the scalar offset.
    int xoff[OPW];
#pragma unroll
    for (int o = 0; o < OPW; ++o) {
        const int pos = 64 * (wave + o * NW) + lane;
        const int r = pos / C;
        xoff[o] = r * D * 2 + ((pos % C) ^ swz<C>(r)) * 16;
    }
    u32x4 xr[OPW];
    auto fetch_x = [&](int b) {
        int side, bh, row0;
        mlp_block(p, nb0, nb1, b, side, bh, row0);
        const MlpSide& sd = p.side[side];
        const uint16_t* xb = (const uint16_t*)sd.x + bh * sd.x_bh_stride + (long long)sd.r0 * D;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)xb, (short)0, (sd.r1 - sd.r0) * D * 2, 0x00020000);  // rows past r1 read as zero
#pragma unroll
        for (int o = 0; o < OPW; ++o)
            xr[o] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, xoff[o], row0 * D * 2, 0));
    };
    auto store_x = [&](lds_u16* dst) {
#pragma unroll
        for (int o = 0; o < OPW; ++o)
            *(__attribute__((address_space(3))) u32x4*)(dst + 512 * (wave + o * NW) + 8 * lane) = xr[o];
    };

    bf16x8 w1f[KS1], w2f[KS2];
    float b1v[16], b2v[16];
    int loaded = -1;  // (side, head) whose weights the registers hold

    fetch_x(b_begin);
    store_x(xs);
    for (int b = b_begin; b < b_end; ++b) {
        int side, bh, row0;
        mlp_block(p, nb0, nb1, b, side, bh, row0);
        const MlpSide& sd = p.side[side];
        const int head = bh % p.H;
        const int key = side * p.H + head;
        if (key != loaded) {
            loaded = key;
            if (wave < HT) {
                const uint16_t* w1 = (const uint16_t*)sd.w1 + ((long long)head * HID + 32 * wave + lq) * D + 8 * h;
#pragma unroll
                for (int s = 0; s < KS1; ++s) w1f[s] = __builtin_bit_cast(bf16x8, ldg_b128(w1 + 16 * s));
                const float* b1 = sd.b1 + (long long)head * HID + 32 * wave + 4 * h;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const f32x4 t = *(const f32x4*)(b1 + 8 * j);
#pragma unroll
                    for (int i = 0; i < 4; ++i) b1v[4 * j + i] = t[i];
                }
            }
            if (wave < FT) {
                const uint16_t* w2 = (const uint16_t*)sd.w2 + ((long long)head * 2 * D + 32 * wave + lq) * HID + 8 * h;
#pragma unroll
                for (int s = 0; s < KS2; ++s) w2f[s] = __builtin_bit_cast(bf16x8, ldg_b128(w2 + 16 * s));
                const float* b2 = sd.b2 + (long long)head * 2 * D + 32 * wave + 4 * h;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const f32x4 t = *(const f32x4*)(b2 + 8 * j);
#pragma unroll
                    for (int i = 0; i < 4; ++i) b2v[4 * j + i] = t[i];
                }
            }
            // the weights are in registers on every path below, so the
            // compiler adds no waits for them
            __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
        }
        // this block's x is in its LDS slot (and every wave is done with the
        // hidden tile and with the x slot written next); the next block's x
        // goes to registers now, to LDS after layer 2
        lds_write_barrier();
        if (b + 1 < b_end) fetch_x(b + 1);
        {
        const lds_u16* xcur = xs + ((b - b_begin) & 1) * XT;

        // layer 1: H^T rows [32 wave, +32) for 4 row tiles
        if (wave < HT) {
#pragma unroll
            for (int rt = 0; rt < RB / 32; ++rt) {
                const int row = 32 * rt + lq;
                f32x16 acc = f32x16{};
#pragma unroll
                for (int s = 0; s < KS1; ++s) {
                    const bf16x8 xf = lds_read_b128(xcur, row * D + (((2 * s + h) ^ swz<C>(row)) << 3));
                    acc = mfma32x32x16(w1f[s], xf, acc);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float y[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) y[i] = fmaxf(acc[4 * j + i] + b1v[4 * j + i], 0.0f);
                    const int c = 4 * wave + j;  // hidden 32 wave + 8 j + 4 h .. + 3: half h of chunk c
                    *(__attribute__((address_space(3))) u32x2*)(hs + row * HID + ((c ^ hswz<CH>(row)) << 3) + 4 * h) =
                        u32x2{pack2_bf16(y[0], y[1]), pack2_bf16(y[2], y[3])};
                }
            }
        }
        }
        lds_write_barrier();  // every wave's hidden rows are in LDS

        // layer 2: psi^T rows [32 wave, +32), phi, store (a resource ending at
        // the side's last row drops the rows past it)
        if (wave < FT) {
            const int nrows = min(sd.r1 - sd.r0 - row0, RB);
            uint16_t* ob = (uint16_t*)sd.out + bh * sd.out_bh_stride + (long long)(sd.r0 + row0) * 2 * D;
            const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(
                (void*)ob, (short)0, nrows * 2 * D * 2, 0x00020000);
            // the wave's feature tile fixes the map (1 + elu for the first
            // half of D', the square for the second): one instance each, so
            // that no element carries a branch
            auto layer2 = [&](auto square_c) {
                constexpr bool SQUARE = decltype(square_c)::value;
#pragma unroll 1
                for (int rt = 0; rt < RB / 32; ++rt) {
                    const int row = 32 * rt + lq;
                    f32x16 acc = f32x16{};
#pragma unroll
                    for (int s = 0; s < KS2; ++s) {
                        const bf16x8 hf = lds_read_b128(hs, row * HID + (((2 * s + h) ^ hswz<CH>(row)) << 3));
                        acc = mfma32x32x16(w2f[s], hf, acc);
                    }
                    // the next block's x into its slot before the first phi store:
                    // the compiler's wait for the x registers would otherwise
                    // include the stores issued after the loads
                    if (rt == 0 && b + 1 < b_end) store_x(xs + ((b + 1 - b_begin) & 1) * XT);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        float y[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float ps = acc[4 * j + i] + b2v[4 * j + i];
                            y[i] = SQUARE ? ps * ps : elu1(ps);
                        }
                        __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack2_bf16(y[0], y[1]), pack2_bf16(y[2], y[3])},
                                                              ors, (row * 2 * D + 32 * wave + 8 * j + 4 * h) * 2, 0, 0);
                    }
                }
            };
            if (wave < FT / 2) layer2(std::false_type{});
            else layer2(std::true_type{});
        } else if (b + 1 < b_end) {
            store_x(xs + ((b + 1 - b_begin) & 1) * XT);
        }
    }
}

// fp32: 32 rows per workgroup of 256 threads; x rows and the hidden layer in LDS.
template <int D>
__global__ __launch_bounds__(256) void phi_mlp_f32_kernel(MlpParams p) {
    constexpr int R = 32;
    __shared__ float xs[R][D];
    __shared__ float hs[R][256];
    const int HID = p.hidden;
    const int tid = threadIdx.x;
    const int nb0 = p.n_sides > 0 ? cdiv(max(p.side[0].r1 - p.side[0].r0, 0), R) : 0;
    const int nb1 = p.n_sides > 1 ? cdiv(max(p.side[1].r1 - p.side[1].r0, 0), R) : 0;
    const int b = blockIdx.x;
    const int n0 = p.BH * nb0;
    const int side = b < n0 ? 0 : 1;
    const int rem = side ? b - n0 : b;
    const int nb = side ? nb1 : nb0;
    const int bh = rem / nb;
    const int row0 = (rem - bh * nb) * R;
    const MlpSide& sd = p.side[side];
    const int head = bh % p.H;
    const int nrows = min(R, sd.r1 - sd.r0 - row0);
    const float* xb = (const float*)sd.x + bh * sd.x_bh_stride + (long long)(sd.r0 + row0) * D;
    for (int e = tid; e < R * D; e += 256) {
        const int r = e / D, c = e % D;
        xs[r][c] = r < nrows ? xb[(long long)r * D + c] : 0.0f;
    }
    __syncthreads();
    const float* w1 = (const float*)sd.w1 + (long long)head * HID * D;
    const float* b1 = sd.b1 + (long long)head * HID;
    for (int e = tid; e < R * HID; e += 256) {
        const int r = e / HID, a = e % HID;
        float acc = b1[a];
        for (int c = 0; c < D; ++c) acc = fmaf(w1[(long long)a * D + c], xs[r][c], acc);
        hs[r][a] = fmaxf(acc, 0.0f);
    }
    __syncthreads();
    const float* w2 = (const float*)sd.w2 + (long long)head * 2 * D * HID;
    const float* b2 = sd.b2 + (long long)head * 2 * D;
    float* ob = (float*)sd.out + bh * sd.out_bh_stride + (long long)(sd.r0 + row0) * 2 * D;
    for (int e = tid; e < R * 2 * D; e += 256) {
        const int r = e / (2 * D), o = e % (2 * D);
        if (r >= nrows) continue;
        float acc = b2[o];
        for (int a = 0; a < HID; ++a) acc = fmaf(w2[(long long)o * HID + a], hs[r][a], acc);
        ob[(long long)r * 2 * D + o] = o < D ? (acc > 0.0f ? acc + 1.0f : expf(acc)) : acc * acc;
    }
}

template <int D>
hipError_t launch_bf16_d(const MlpParams& p, hipStream_t s) {
    switch (p.hidden) {
    case 32: phi_mlp_bf16_kernel<D, 32><<<p.grid, kMlpRows * 4, 0, s>>>(p); break;
    case 64: phi_mlp_bf16_kernel<D, 64><<<p.grid, kMlpRows * 4, 0, s>>>(p); break;
    case 128: phi_mlp_bf16_kernel<D, 128><<<p.grid, kMlpRows * 4, 0, s>>>(p); break;
    case 256: phi_mlp_bf16_kernel<D, 256><<<p.grid, kMlpRows * 4, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

bool phi_mlp_hidden_ok(int hidden) { return hidden == 32 || hidden == 64 || hidden == 128 || hidden == 256; }

hipError_t launch_phi_mlp_bf16(const MlpParams& p, hipStream_t s) {
    if (p.grid <= 0) return hipSuccess;
    switch (p.d) {
    case 32: return launch_bf16_d<32>(p, s);
    case 64: return launch_bf16_d<64>(p, s);
    case 128: return launch_bf16_d<128>(p, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_phi_mlp_f32(const MlpParams& p, hipStream_t s) {
    long long blocks = 0;
    for (int i = 0; i < p.n_sides; ++i)
        blocks += (long long)p.BH * ((std::max(p.side[i].r1 - p.side[i].r0, 0) + 31) / 32);
    if (blocks <= 0) return hipSuccess;
    if (!phi_mlp_hidden_ok(p.hidden)) return hipErrorInvalidValue;
    switch (p.d) {
    case 16: phi_mlp_f32_kernel<16><<<(unsigned)blocks, 256, 0, s>>>(p); break;
    case 32: phi_mlp_f32_kernel<32><<<(unsigned)blocks, 256, 0, s>>>(p); break;
    case 64: phi_mlp_f32_kernel<64><<<(unsigned)blocks, 256, 0, s>>>(p); break;
    case 128: phi_mlp_f32_kernel<128><<<(unsigned)blocks, 256, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace rehyat
