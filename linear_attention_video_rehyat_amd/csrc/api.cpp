// api.cpp -- the C ABI of librehyat: argument validation, chunk geometry,
// workspace management and launch sequencing.  See include/rehyat.h.
//
// Geometry (ReHyAt, arXiv 2601.04342, §3.3 equation; N' = T_c HW): chunk t owns
// frames [t T_c, min((t+1) T_c, F)); its softmax window starts T_o frames
// earlier (clipped at 0); its linear set is every key before the window.  The
// keys leaving the window between chunk u and u+1 form the delta block
// E_u = frames [max(u T_c - T_o, 0), max((u+1) T_c - T_o, 0)), so the state of
// chunk t is the sum over u < t of the block sums (the chunk-wise RNN form).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <map>
#include <memory>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/rehyat.h"
#include "api_internal.h"
#include "kernels.h"

using namespace rehyat;

namespace {

thread_local std::string g_last_error;
thread_local hipEvent_t g_prof[4] = {nullptr, nullptr, nullptr, nullptr};

// Fault injection (test hook, rehyat_debug_inject_hip_error): every HIP
// runtime call and kernel launch an entry point makes is one "HIP step",
// counted per call on the calling thread.  When armed, step g_inject_at of the
// next call that reaches it fails with REHYAT_EHIP instead of being made; the
// hook then disarms itself.
thread_local int g_inject_at = -1;
thread_local int g_steps = 0;
thread_local bool g_injected = false;

// Start of an entry point's GPU work: clear the last error and the step count.
void begin_call() {
    g_last_error.clear();
    g_steps = 0;
    g_injected = false;
}

template <class Fn>
hipError_t hip_step(Fn&& fn) {
    const int i = g_steps++;
    if (i == g_inject_at) {
        g_inject_at = -1;
        g_injected = true;
        return hipErrorLaunchFailure;
    }
    return fn();
}

hipError_t prof_mark(int i, hipStream_t s) {
    return g_prof[i] ? hip_step([&] { return hipEventRecord(g_prof[i], s); }) : hipSuccess;
}

rehyat_status fail(rehyat_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

rehyat_status hip_fail(hipError_t e, const char* what) {
    if (g_injected)
        return fail(REHYAT_EHIP, "%s: injected failure at HIP step %d (rehyat_debug_inject_hip_error)", what,
                    g_steps - 1);
    return fail(REHYAT_EHIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kStateSubRows = 1024;      // key rows per fp32 block-state workgroup
constexpr int kStateSubRowsBf16 = 1600;  // key rows per bf16 block-state workgroup (25 tiles of 64)

// Split of each delta block (at most `rows` keys) into sub-blocks, one
// workgroup and one partial sum each.  The split depends on the row count
// only, so a streaming step that folds the same rows as a forward delta block
// adds the same partials in the same order (the two results are bitwise
// equal).  The bf16 size gives 3 workgroups per 3-frame block of 1560-token
// frames: 204 workgroups for 12 heads at 21 frames, T_c = 3, T_o = 1 (one
// 2-frame block of 2 sub-blocks and five 3-frame blocks of 3).
struct SubSplit {
    int n_sub, sub_rows;
};
SubSplit state_split(int dtype, long long rows) {
    const int sub = dtype == REHYAT_BF16 ? kStateSubRowsBf16 : kStateSubRows;
    const long long n = (std::max<long long>(rows, 1) + sub - 1) / sub;
    return {(int)n, sub};
}

// Workgroups per (b, h) of a block-state launch: the sub-blocks of every block.
int state_items_per_bh(const StateParams& sp) {
    const BlockPart part = state_part(sp);
    int n = 0;
    for (int u = 0; u < sp.n_blocks; ++u) n += part_block_subs(part, u);
    return n;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool bf16_dim_ok(int d) { return d == 32 || d == 64 || d == 128; }
bool f32_dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

struct Geometry {
    int B, H, F, HW, d, Tc, To, phi, dtype;
    long long N;      // tokens per (b, h)
    int BH, C, Dp, E; // chunks, feature dim, state elements (d*Dp + Dp)
    int elem;         // bytes per element of q/k/v/out
};

rehyat_status check_common(Geometry& g, int B, int H, int frames, int tpf, int d, int Tc, int To,
                           int phi, int dtype, bool mlp = false) {
    if (B < 1 || H < 1) return fail(REHYAT_EINVAL, "B and H must be >= 1 (got B=%d H=%d)", B, H);
    if (frames < 1 || tpf < 1)
        return fail(REHYAT_EINVAL, "frames and tokens_per_frame must be >= 1 (got %d, %d)", frames, tpf);
    if (Tc < 1) return fail(REHYAT_EINVAL, "chunk_frames must be >= 1 (got %d)", Tc);
    if (To < 0) return fail(REHYAT_EINVAL, "overlap_frames must be >= 0 (got %d)", To);
    if (phi < REHYAT_PHI_NONE || phi > REHYAT_PHI_MLP2)
        return fail(REHYAT_EINVAL, "unknown feature_map %d", phi);
    if ((phi == REHYAT_PHI_MLP2) != mlp)
        return fail(REHYAT_EINVAL, mlp ? "internal: learned map without REHYAT_PHI_MLP2"
                                       : "REHYAT_PHI_MLP2 needs its weights: use the _mlp entry points");
    if (dtype != REHYAT_F32 && dtype != REHYAT_BF16) return fail(REHYAT_EINVAL, "unknown dtype %d", dtype);
    if (dtype == REHYAT_BF16 && !bf16_dim_ok(d))
        return fail(REHYAT_EUNSUPPORTED, "head_dim %d not supported for bf16 (32, 64, 128)", d);
    if (dtype == REHYAT_F32 && !f32_dim_ok(d))
        return fail(REHYAT_EUNSUPPORTED, "head_dim %d not supported for fp32 (16, 32, 64, 128)", d);
    const long long N = (long long)frames * tpf;
    if (N > (1LL << 30)) return fail(REHYAT_EINVAL, "frames*tokens_per_frame = %lld is too large", N);
    // the kernels address the rows of one (b, h) through buffer resources with
    // 32-bit byte offsets: every per-(b, h) extent (input rows, and the learned
    // map's 2 head_dim-wide feature rows) must stay below 2^31 bytes
    const long long row_bytes = (long long)(mlp ? 2 * d : d) * (dtype == REHYAT_BF16 ? 2 : 4);
    if (N * row_bytes >= (1LL << 31))
        return fail(REHYAT_EUNSUPPORTED,
                    "frames*tokens_per_frame = %lld is too large: %lld bytes of rows per (b, h) exceed the "
                    "2^31-byte extent the kernels address", N, N * row_bytes);
    const long long BH = (long long)B * H;
    if (BH > (1LL << 24)) return fail(REHYAT_EINVAL, "B*H = %lld is too large", BH);
    g.B = B; g.H = H; g.F = frames; g.HW = tpf; g.d = d; g.Tc = Tc; g.To = To; g.phi = phi; g.dtype = dtype;
    g.N = N;
    g.BH = (int)BH;
    g.C = (frames + Tc - 1) / Tc;
    g.Dp = feature_dim(phi, d);
    g.E = d * g.Dp + g.Dp;
    g.elem = dtype == REHYAT_BF16 ? 2 : 4;
    return REHYAT_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

// ---------------------------------------------------------------- local-kernel dispatch order
// The local kernel's workgroups differ in cost (chunk 0 streams a shorter
// window).  Simulate the dispatcher -- each XCD hands its workgroups, in order,
// to whichever of its CUs frees up first -- for the natural and the
// longest-first order of each XCD's items (local_work_item), and keep the
// longest-first order where it finishes earlier.  Decisions are cached per
// geometry.
long long local_makespan(const LocalParams& lp, int blocks, int bn, int cus_per_xcd) {
    long long worst = 0;
    std::vector<long long> cu(cus_per_xcd);
    for (int x = 0; x < 8; ++x) {
        std::fill(cu.begin(), cu.end(), 0);
        for (int bid = x; bid < blocks; bid += 8) {
            const int item = local_work_item(lp, bid, blocks, bn);
            const int t = (item / lp.tiles_per_chunk) % lp.n_chunks;
            auto it = std::min_element(cu.begin(), cu.end());
            *it += chunk_key_tiles(lp, t, bn) + 2;  // + the epilogue, about two key tiles
        }
        worst = std::max(worst, *std::max_element(cu.begin(), cu.end()));
    }
    return worst;
}

int cus_per_xcd() {
    static std::mutex mu;
    static std::vector<int> per_dev;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 32;
    std::lock_guard<std::mutex> lock(mu);
    if ((int)per_dev.size() <= dev) per_dev.resize(dev + 1, 0);
    if (per_dev[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 8) n = 256;
        per_dev[dev] = n / 8;
    }
    return per_dev[dev];
}

int choose_lpt_order(const LocalParams& lp, int blocks, int bn) {
    if (lp.n_chunks < 2 || blocks < 16) return 0;
    const int cpx = cus_per_xcd();
    static std::mutex mu;
    static std::map<std::vector<long long>, int> cache;
    const std::vector<long long> key = {lp.BH, lp.n_chunks, lp.tiles_per_chunk, lp.F, lp.Tc, lp.To, lp.HW,
                                        lp.prev_rows, bn, cpx, blocks};
    {
        std::lock_guard<std::mutex> lock(mu);
        auto f = cache.find(key);
        if (f != cache.end()) return f->second;
    }
    LocalParams a = lp, b = lp;
    a.lpt_order = 0;
    b.lpt_order = 1;
    const int use = local_makespan(b, blocks, bn, cpx) < local_makespan(a, blocks, bn, cpx) ? 1 : 0;
    std::lock_guard<std::mutex> lock(mu);
    cache[key] = use;
    return use;
}

// ---------------------------------------------------------------- workspace arenas
// One arena per (device, stream): calls queued on different streams never
// share workspace, so they may run concurrently.  A lease holds its arena's
// lock from the moment a call takes the workspace until the call's last launch
// is queued; a concurrent call on the same stream from another thread waits
// rather than growing (and freeing) the buffer under it.  Growing waits for the
// stream's queued work, the only work that can still use the old buffer.
struct Arena {
    std::mutex mu;
    void* ptr = nullptr;
    size_t bytes = 0;
};
std::mutex g_arenas_mu;
std::map<std::pair<int, uintptr_t>, std::unique_ptr<Arena>> g_arenas;

struct ArenaLease {
    std::unique_lock<std::mutex> lock;
    char* ptr = nullptr;
};

rehyat_status arena_acquire(size_t bytes, hipStream_t s, ArenaLease& lease) {
    int dev = 0;
    hipError_t e = hip_step([&] { return hipGetDevice(&dev); });
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    Arena* a = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_arenas_mu);
        std::unique_ptr<Arena>& slot = g_arenas[{dev, (uintptr_t)s}];
        if (!slot) slot.reset(new Arena());
        a = slot.get();
    }
    std::unique_lock<std::mutex> lock(a->mu);
    if (a->bytes < bytes) {
        if (a->ptr) {
            e = hip_step([&] { return hipStreamSynchronize(s); });
            if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
            (void)hipFree(a->ptr);
            a->ptr = nullptr;
            a->bytes = 0;
        }
        const size_t want = bytes + bytes / 4 + (1u << 20);
        e = hip_step([&] { return hipMalloc(&a->ptr, want); });
        if (e != hipSuccess) {
            (void)hipGetLastError();
            a->ptr = nullptr;
            if (g_injected) return hip_fail(e, "hipMalloc");
            return fail(REHYAT_ENOMEM, "cannot allocate %zu bytes of workspace: %s", want, hipGetErrorString(e));
        }
        a->bytes = want;
    }
    lease.ptr = (char*)a->ptr;
    lease.lock = std::move(lock);
    return REHYAT_OK;
}

// Waits for the stream's queued work and frees its arena on the current device.
rehyat_status arena_release(hipStream_t s) {
    int dev = 0;
    hipError_t e = hip_step([&] { return hipGetDevice(&dev); });
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::unique_ptr<Arena> a;
    {
        std::lock_guard<std::mutex> lock(g_arenas_mu);
        auto it = g_arenas.find({dev, (uintptr_t)s});
        if (it == g_arenas.end()) return REHYAT_OK;
        std::lock_guard<std::mutex> alock(it->second->mu);  // no call holds a lease on it now
        a = std::move(it->second);
        g_arenas.erase(it);
    }
    if (a->ptr) {
        e = hip_step([&] { return hipStreamSynchronize(s); });
        if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
        (void)hipFree(a->ptr);
    }
    return REHYAT_OK;
}

// Side streams.  A streaming step's local-attention launch covers one chunk
// (228 workgroups at the Wan shape, fewer than the 256 CUs), and the state
// update that the next step needs (fold, scan, overlap copy) reads only the
// step's inputs, so it runs beside the local launch on a library-owned stream:
// an event recorded on the caller's stream forks it, an event recorded on it
// joins the caller's stream back.  One per (device, caller stream), created on
// first use and kept until rehyat_workspace_release for that stream; its lock
// is held while a call queues work on it.
struct SideStream {
    std::mutex mu;
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_sides_mu;
std::map<std::pair<int, uintptr_t>, std::unique_ptr<SideStream>> g_sides;

struct SideLease {
    std::unique_lock<std::mutex> lock;
    SideStream* side = nullptr;
};

void side_destroy(SideStream& ss) {
    if (ss.s) (void)hipStreamSynchronize(ss.s);
    if (ss.join) (void)hipEventDestroy(ss.join);
    if (ss.fork) (void)hipEventDestroy(ss.fork);
    if (ss.s) (void)hipStreamDestroy(ss.s);
    ss.s = nullptr;
    ss.fork = ss.join = nullptr;
}

rehyat_status side_acquire(hipStream_t s, SideLease& lease) {
    int dev = 0;
    hipError_t e = hip_step([&] { return hipGetDevice(&dev); });
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    SideStream* ss = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_sides_mu);
        std::unique_ptr<SideStream>& slot = g_sides[{dev, (uintptr_t)s}];
        if (!slot) slot.reset(new SideStream());
        ss = slot.get();
    }
    std::unique_lock<std::mutex> lock(ss->mu);
    if (!ss->s) {
        e = hip_step([&] { return hipStreamCreateWithFlags(&ss->s, hipStreamNonBlocking); });
        if (e == hipSuccess) e = hip_step([&] { return hipEventCreateWithFlags(&ss->fork, hipEventDisableTiming); });
        if (e == hipSuccess) e = hip_step([&] { return hipEventCreateWithFlags(&ss->join, hipEventDisableTiming); });
        if (e != hipSuccess) {
            side_destroy(*ss);
            return hip_fail(e, "side stream creation");
        }
    }
    lease.side = ss;
    lease.lock = std::move(lock);
    return REHYAT_OK;
}

// Waits for the side stream's work and destroys it (current device).
void side_release(hipStream_t s) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return;
    std::unique_ptr<SideStream> ss;
    {
        std::lock_guard<std::mutex> lock(g_sides_mu);
        auto it = g_sides.find({dev, (uintptr_t)s});
        if (it == g_sides.end()) return;
        std::lock_guard<std::mutex> slock(it->second->mu);
        ss = std::move(it->second);
        g_sides.erase(it);
    }
    side_destroy(*ss);
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace of the whole-clip forward: partial block sums and prepared states.
struct FwdWorkspace {
    size_t partial_off, shi_off, slo_off, z_off, suffix_off, fq_off, fk_off, total;
    int U, n_sub;
    SubSplit split;
};

FwdWorkspace fwd_workspace(const Geometry& g, int mode) {
    FwdWorkspace w{};
    w.U = state_block_count(mode, g.C);
    // longest block: T_c frames (recurrent form); max(r, T_c - r) frames with
    // r = T_o mod T_c, or T_c when r = 0 (bidirectional form)
    long long block_frames = g.Tc;
    if (mode == kBidirectional && g.To % g.Tc != 0) block_frames = std::max(g.To % g.Tc, g.Tc - g.To % g.Tc);
    w.split = state_split(g.dtype, block_frames * g.HW);
    w.n_sub = w.split.n_sub;
    const size_t partial = (size_t)g.BH * w.U * w.n_sub * g.E * 4;
    const size_t sprep = (size_t)g.BH * g.C * g.d * g.Dp * (g.dtype == REHYAT_BF16 ? 2 : 4);
    const size_t zprep = (size_t)g.BH * g.C * g.Dp * 4;
    w.partial_off = 0;
    w.shi_off = align256(partial);
    w.slo_off = w.shi_off + align256(sprep);
    w.z_off = w.slo_off + (g.dtype == REHYAT_BF16 ? align256(sprep) : 0);
    w.suffix_off = w.z_off + align256(zprep);
    const size_t suffix = mode == kBidirectional ? (size_t)g.BH * g.C * g.E * 4 : 0;
    // learned map: phi(q) and phi(k) rows, [BH][N][2d] each
    const size_t feat = g.phi == REHYAT_PHI_MLP2 ? (size_t)g.BH * g.N * g.Dp * g.elem : 0;
    w.fq_off = w.suffix_off + align256(suffix);
    w.fk_off = w.fq_off + align256(feat);
    w.total = w.fk_off + align256(feat);
    return w;
}

// Recurrent form: chunk t has a linear set iff t T_c - T_o > 0 (the last chunk
// is t = C-1).  Bidirectional form: every chunk's window misses some key as
// soon as there are two chunks.
bool any_linear(const Geometry& g, int mode) {
    if (g.phi == REHYAT_PHI_NONE) return false;
    if (mode == kBidirectional) return g.C >= 2;
    return (long long)(g.C - 1) * g.Tc - g.To > 0;
}

// The learned feature map of rows [rq0, rq1) of x_q and [rk0, rk1) of x_k
// (every (b, h)) into fq / fk, laid out like the inputs with 2d columns.
hipError_t launch_mlp(const Geometry& g, const rehyat_mlp_weights* wq, const rehyat_mlp_weights* wk,
                      const void* xq, void* fq, long long q_rows, int rq0, int rq1,
                      const void* xk, void* fk, long long k_rows, int rk0, int rk1, hipStream_t s) {
    MlpParams mp{};
    const rehyat_mlp_weights* ws[2] = {wq, wk};
    const void* xs[2] = {xq, xk};
    void* os[2] = {fq, fk};
    const long long rows[2] = {q_rows, k_rows};
    const int r0[2] = {rq0, rk0}, r1[2] = {rq1, rk1};
    for (int i = 0; i < 2; ++i) {
        if (r1[i] <= r0[i]) continue;
        MlpSide& sd = mp.side[mp.n_sides++];
        sd.x = xs[i]; sd.out = os[i];
        sd.w1 = ws[i]->w1; sd.b1 = ws[i]->b1; sd.w2 = ws[i]->w2; sd.b2 = ws[i]->b2;
        sd.x_bh_stride = rows[i] * g.d; sd.out_bh_stride = rows[i] * g.Dp;
        sd.r0 = r0[i]; sd.r1 = r1[i];
    }
    if (mp.n_sides == 0) return hipSuccess;
    mp.BH = g.BH; mp.H = g.H; mp.d = g.d; mp.hidden = wq->hidden;
    if (g.dtype == REHYAT_BF16) {
        long long blocks = 0;
        for (int i = 0; i < mp.n_sides; ++i) blocks += (long long)g.BH * ((mp.side[i].r1 - mp.side[i].r0 + 127) / 128);
        mp.grid = (int)std::min<long long>(blocks, 8LL * cus_per_xcd());
        return launch_phi_mlp_bf16(mp, s);
    }
    return launch_phi_mlp_f32(mp, s);
}

// Query rows whose chunk has a linear set, and key rows in some linear set.
void mlp_rows(const Geometry& g, int mode, int& q0, int& k1) {
    if (mode == kBidirectional) {
        q0 = 0;
        k1 = (int)g.N;
        return;
    }
    const long long t_min = g.To / g.Tc + 1;  // first chunk with t T_c - T_o > 0
    q0 = (int)(std::min<long long>(t_min * g.Tc, g.F) * g.HW);
    k1 = (int)(std::max<long long>((long long)(g.C - 1) * g.Tc - g.To, 0) * g.HW);
}

// Bytes of workspace a whole-clip forward needs (0 when no chunk has a linear set).
size_t fwd_workspace_bytes(const Geometry& g, int mode) {
    return any_linear(g, mode) ? fwd_workspace(g, mode).total : 0;
}

// The launches of a whole-clip forward, with its workspace at `ws`
// (fwd_workspace_bytes(g, mode) bytes; null when that is 0).
rehyat_status run_fwd_ws(const void* q, const void* k, const void* v, void* out, const Geometry& g, int mode,
                         float* pm, float* pnt, float* poS, float* poL, float* pnL, hipStream_t s,
                         const rehyat_mlp_weights* wq, const rehyat_mlp_weights* wk, float* lse, float* out_f32,
                         char* ws) {
    const bool lin = any_linear(g, mode);
    FwdWorkspace w{};
    hipError_t pe = prof_mark(0, s);
    if (pe != hipSuccess) return hip_fail(pe, "hipEventRecord");
    if (lin) {
        w = fwd_workspace(g, mode);
        if (!ws) return fail(REHYAT_EINVAL, "internal: forward without its workspace");
        if (g.phi == REHYAT_PHI_MLP2) {
            int q0 = 0, k1 = 0;
            mlp_rows(g, mode, q0, k1);
            hipError_t e = hip_step([&] { return launch_mlp(g, wq, wk, q, ws + w.fq_off, g.N, q0, (int)g.N, k, ws + w.fk_off, g.N, 0, k1, s); });
            if (e != hipSuccess) return hip_fail(e, "feature-map launch");
        }

        StateParams sp{};
        sp.k = k; sp.v = v; sp.kp = nullptr; sp.vp = nullptr;
        sp.bh_stride = g.N * g.d; sp.prev_bh_stride = 0; sp.prev_rows = 0;
        sp.HW = g.HW; sp.Tc = g.Tc; sp.To = g.To;
        sp.n_blocks = w.U; sp.sub_rows = w.split.sub_rows; sp.n_sub = w.n_sub; sp.stream_rows = 0;
        sp.BH = g.BH; sp.d = g.d; sp.phi = g.phi;
        sp.mode = mode; sp.F = g.F;
        sp.partial = (float*)(ws + w.partial_off);
        if (g.phi == REHYAT_PHI_MLP2) {
            sp.fk = ws + w.fk_off; sp.fk_bh_stride = g.N * g.Dp;
            sp.fkp = nullptr; sp.fkp_bh_stride = 0;
        }
        sp.items_per_bh = state_items_per_bh(sp);
        hipError_t e = hip_step([&] { return g.dtype == REHYAT_BF16 ? launch_state_bf16(sp, s) : launch_state_f32(sp, s); });
        if (e != hipSuccess) return hip_fail(e, "block-state launch");
        if ((e = prof_mark(1, s)) != hipSuccess) return hip_fail(e, "hipEventRecord");

        ScanParams cp{};
        cp.partial = sp.partial; cp.part = state_part(sp); cp.init = nullptr; cp.state_out = nullptr;
        cp.s_hi = ws + w.shi_off; cp.s_lo = ws + w.slo_off; cp.z = (float*)(ws + w.z_off);
        cp.s_chunk_stride = (long long)g.d * g.Dp; cp.s_bh_stride = (long long)g.C * g.d * g.Dp;
        cp.z_chunk_stride = g.Dp; cp.z_bh_stride = (long long)g.C * g.Dp;
        cp.U = w.U; cp.n_sub = w.n_sub; cp.BH = g.BH; cp.d = g.d; cp.Dp = g.Dp;
        cp.t_first = mode == kBidirectional ? 0 : 1; cp.t_offset = 0; cp.f32_prep = g.dtype == REHYAT_F32;
        cp.mode = mode; cp.C = g.C; cp.q = g.To / g.Tc;
        cp.suffix = mode == kBidirectional ? (float*)(ws + w.suffix_off) : nullptr;
        e = hip_step([&] { return launch_scan(cp, s); });
        if (e != hipSuccess) return hip_fail(e, "scan launch");
    } else {
        if ((pe = prof_mark(1, s)) != hipSuccess) return hip_fail(pe, "hipEventRecord");
    }
    if ((pe = prof_mark(2, s)) != hipSuccess) return hip_fail(pe, "hipEventRecord");
    LocalParams lp{};
    lp.q = q; lp.out = out; lp.k = k; lp.v = v; lp.kp = nullptr; lp.vp = nullptr;
    lp.bh_stride = g.N * g.d; lp.prev_bh_stride = 0; lp.prev_rows = 0;
    lp.HW = g.HW; lp.F = g.F; lp.Tc = g.Tc; lp.To = g.To;
    lp.n_chunks = g.C; lp.BH = g.BH; lp.d = g.d;
    const int bm = g.dtype == REHYAT_BF16 ? local_bf16_tile_rows(g.d) : local_f32_tile_rows(g.d);
    const long long rows_per_chunk = (long long)std::min<long long>(g.Tc, g.F) * g.HW;
    lp.tiles_per_chunk = (int)((rows_per_chunk + bm - 1) / bm);
    const long long blocks = (long long)g.BH * g.C * lp.tiles_per_chunk;
    if (blocks > 0x7fffffffLL) return fail(REHYAT_EINVAL, "problem too large: %lld workgroups", blocks);
    lp.phi = g.phi; lp.lin_always = mode == kBidirectional ? 1 : 0;
    lp.lpt_order = g.dtype == REHYAT_BF16 ? choose_lpt_order(lp, (int)blocks, local_bf16_key_tile(g.d)) : 0;
    if (lin) {
        lp.s_hi = ws + w.shi_off; lp.s_lo = ws + w.slo_off; lp.z = (const float*)(ws + w.z_off);
        lp.s_chunk_stride = (long long)g.d * g.Dp; lp.s_bh_stride = (long long)g.C * g.d * g.Dp;
        lp.z_chunk_stride = g.Dp; lp.z_bh_stride = (long long)g.C * g.Dp;
        if (g.phi == REHYAT_PHI_MLP2) {
            lp.fq = ws + w.fq_off;
            lp.fq_bh_stride = g.N * g.Dp;
        }
    } else {
        lp.phi = REHYAT_PHI_NONE;  // no chunk has a linear set
    }
    lp.pm = pm; lp.pnt = pnt; lp.poS = poS; lp.poL = poL; lp.pnL = pnL;
    lp.lse = lse;
    lp.out_f32 = g.dtype == REHYAT_BF16 ? out_f32 : nullptr;
    hipError_t e = hip_step([&] { return g.dtype == REHYAT_BF16 ? launch_local_bf16(lp, s) : launch_local_f32(lp, s); });
    if (e != hipSuccess) return hip_fail(e, "local-attention launch");
    if ((e = prof_mark(3, s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    return REHYAT_OK;
}

// A whole-clip forward with its workspace from the stream's arena.
rehyat_status run_fwd(const void* q, const void* k, const void* v, void* out, const Geometry& g, int mode,
                      float* pm, float* pnt, float* poS, float* poL, float* pnL, hipStream_t s,
                      const rehyat_mlp_weights* wq = nullptr, const rehyat_mlp_weights* wk = nullptr,
                      float* lse = nullptr, float* out_f32 = nullptr) {
    ArenaLease lease;
    const size_t need = fwd_workspace_bytes(g, mode);
    if (need) {
        const rehyat_status st = arena_acquire(need, s, lease);
        if (st != REHYAT_OK) return st;
    }
    return run_fwd_ws(q, k, v, out, g, mode, pm, pnt, poS, poL, pnL, s, wq, wk, lse, out_f32, lease.ptr);
}

// Weights of the learned query and key maps: present, 16-byte aligned, and a
// hidden width the kernels are built for (the same for both maps).
rehyat_status check_mlp(const rehyat_mlp_weights* wq, const rehyat_mlp_weights* wk) {
    if (!wq || !wk) return fail(REHYAT_EINVAL, "null feature-map weights");
    for (const rehyat_mlp_weights* w : {wq, wk}) {
        if (!w->w1 || !w->b1 || !w->w2 || !w->b2) return fail(REHYAT_EINVAL, "null feature-map weight pointer");
        if (!aligned16(w->w1) || !aligned16(w->b1) || !aligned16(w->w2) || !aligned16(w->b2))
            return fail(REHYAT_EINVAL, "feature-map weights must be 16-byte aligned");
        if (!phi_mlp_hidden_ok(w->hidden))
            return fail(REHYAT_EUNSUPPORTED, "feature-map hidden width %d not supported (32, 64, 128, 256)", w->hidden);
    }
    if (wq->hidden != wk->hidden)
        return fail(REHYAT_EUNSUPPORTED, "query and key maps must have the same hidden width (%d vs %d)",
                    wq->hidden, wk->hidden);
    return REHYAT_OK;
}

// fixed_ws: the workspace is the device buffer it supplies, fixed_bytes bytes,
// instead of the stream's arena (REHYAT_ENOMEM if the call needs more).
rehyat_status fwd_entry(const void* q, const void* k, const void* v, void* out, int B, int H,
                        int frames, int tpf, int d, int Tc, int To, int phi, int dtype, int mode,
                        void* stream, const rehyat_mlp_weights* wq = nullptr,
                        const rehyat_mlp_weights* wk = nullptr, fixed_workspace_fn fixed_ws = nullptr,
                        size_t fixed_bytes = 0) {
    Geometry g{};
    const bool mlp = phi == REHYAT_PHI_MLP2 && (wq || wk);
    rehyat_status st = check_common(g, B, H, frames, tpf, d, Tc, To, phi, dtype, mlp);
    if (st != REHYAT_OK) return st;
    if (mlp && (st = check_mlp(wq, wk)) != REHYAT_OK) return st;
    if (!q || !k || !v || !out) return fail(REHYAT_EINVAL, "null tensor pointer");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(REHYAT_EINVAL, "tensor pointers must be 16-byte aligned");
    const size_t bytes = (size_t)g.BH * g.N * g.d * g.elem;
    if (overlaps(out, bytes, q, bytes) || overlaps(out, bytes, k, bytes) || overlaps(out, bytes, v, bytes))
        return fail(REHYAT_EINVAL, "out must not overlap q, k or v");
    if (fixed_ws) {
        const size_t need = fwd_workspace_bytes(g, mode);
        if (need > fixed_bytes)
            return fail(REHYAT_ENOMEM, "the call needs %zu bytes of workspace; the fixed scratch holds %zu",
                        need, fixed_bytes);
        begin_call();
        char* ws = nullptr;
        if (need) {  // the buffer's address: one HIP step (a runtime lookup)
            rehyat_status wst = REHYAT_OK;
            const hipError_t e = hip_step([&] {
                wst = fixed_ws(&ws);
                return wst == REHYAT_OK ? hipSuccess : hipErrorInvalidSymbol;
            });
            if (g_injected) return hip_fail(e, "fixed workspace lookup");
            if (wst != REHYAT_OK) return wst;
        }
        return run_fwd_ws(q, k, v, out, g, mode, nullptr, nullptr, nullptr, nullptr, nullptr, (hipStream_t)stream,
                          wq, wk, nullptr, nullptr, ws);
    }
    begin_call();
    return run_fwd(q, k, v, out, g, mode, nullptr, nullptr, nullptr, nullptr, nullptr, (hipStream_t)stream, wq, wk);
}

rehyat_status partials_entry(const void* q, const void* k, const void* v, int dtype, float* m, float* nt,
                             float* o_s, float* o_l, float* n_l, int B, int H, int frames, int tpf, int d,
                             int Tc, int To, int phi, int mode, void* stream,
                             const rehyat_mlp_weights* wq = nullptr, const rehyat_mlp_weights* wk = nullptr) {
    Geometry g{};
    const bool mlp = phi == REHYAT_PHI_MLP2 && (wq || wk);
    rehyat_status st = check_common(g, B, H, frames, tpf, d, Tc, To, phi, dtype, mlp);
    if (st != REHYAT_OK) return st;
    if (mlp && (st = check_mlp(wq, wk)) != REHYAT_OK) return st;
    if (!q || !k || !v) return fail(REHYAT_EINVAL, "null tensor pointer");
    if (!m && !nt && !o_s && !o_l && !n_l) return fail(REHYAT_EINVAL, "no partial output requested");
    const void* ptrs[8] = {q, k, v, m, nt, o_s, o_l, n_l};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return fail(REHYAT_EINVAL, "pointers must be 16-byte aligned");
    begin_call();
    return run_fwd(q, k, v, nullptr, g, mode, m, nt, o_s, o_l, n_l, (hipStream_t)stream, wq, wk);
}

// ---------------------------------------------------------------- backward
// Workspace of the backward: dsum, the forward's prepared states (both
// layouts), and the gradient sums per chunk-row block with their suffix (or,
// bidirectional, prefix + suffix) combinations per key block.
struct BwdWorkspace {
    size_t dsum_off, part_off, shi_off, slo_off, thi_off, tlo_off, z_off, suffix_off;
    size_t gpart_off, ghi_off, glo_off, gthi_off, gtlo_off, gz_off, gsuffix_off, total;
    int U, GU, gslots;
    SubSplit split, gsplit;
};

BwdWorkspace bwd_workspace(const Geometry& g, int mode) {
    BwdWorkspace w{};
    const bool bf = g.dtype == REHYAT_BF16;
    const bool bidir = mode == kBidirectional;
    w.U = state_block_count(mode, g.C);                          // forward blocks
    w.GU = bidir ? g.C : std::max(g.C - 1, 0);                   // chunk-row blocks
    w.gslots = bidir ? 2 * g.C + 1 : g.C;                        // gradient sums per key block
    long long block_frames = g.Tc;
    if (bidir && g.To % g.Tc != 0) block_frames = std::max(g.To % g.Tc, g.Tc - g.To % g.Tc);
    w.split = state_split(g.dtype, block_frames * g.HW);
    w.gsplit = state_split(g.dtype, (long long)g.Tc * g.HW);    // a chunk: at most T_c frames
    const size_t prep = (size_t)g.BH * g.C * g.d * g.Dp * (bf ? 2 : 4);
    const size_t gprep = (size_t)g.BH * w.gslots * g.d * g.Dp * (bf ? 2 : 4);
    size_t off = 0;
    auto take = [&](size_t bytes) { const size_t o = off; off += align256(bytes); return o; };
    w.dsum_off = take((size_t)g.BH * g.N * 4);
    w.part_off = take((size_t)g.BH * w.U * w.split.n_sub * g.E * 4);
    w.shi_off = take(prep);
    w.slo_off = take(bf ? prep : 0);
    w.thi_off = take(prep);
    w.tlo_off = take(bf ? prep : 0);
    w.z_off = take((size_t)g.BH * g.C * g.Dp * 4);
    w.suffix_off = take(bidir ? (size_t)g.BH * g.C * g.E * 4 : 0);
    w.gpart_off = take((size_t)g.BH * w.GU * w.gsplit.n_sub * g.E * 4);
    w.ghi_off = take(gprep);
    w.glo_off = take(bf ? gprep : 0);
    w.gthi_off = take(gprep);
    w.gtlo_off = take(bf ? gprep : 0);
    w.gz_off = take((size_t)g.BH * w.gslots * g.Dp * 4);
    w.gsuffix_off = take(bidir ? (size_t)g.BH * (g.C + 1) * g.E * 4 : 0);
    w.total = off;
    return w;
}

rehyat_status bwd_entry(const void* q, const void* k, const void* v, const void* out, const float* out_f32,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv, int dtype, int B,
                        int H, int frames, int tpf, int d, int Tc, int To, int phi, int mode, void* stream) {
    Geometry g{};
    rehyat_status st = check_common(g, B, H, frames, tpf, d, Tc, To, phi, dtype);
    if (st != REHYAT_OK) return st;
    const void* ins[6] = {q, k, v, out, lse, dout};
    void* outs[3] = {dq, dk, dv};
    for (const void* x : ins)
        if (!x || !aligned16(x)) return fail(REHYAT_EINVAL, "null or misaligned input pointer");
    for (void* x : outs)
        if (!x || !aligned16(x)) return fail(REHYAT_EINVAL, "null or misaligned gradient pointer");
    const size_t bytes = (size_t)g.BH * g.N * g.d * g.elem;
    if (out_f32 && !aligned16(out_f32)) return fail(REHYAT_EINVAL, "misaligned out_f32");
    for (int a = 0; a < 3; ++a) {
        for (int b = 0; b < 6; ++b)
            if (overlaps(outs[a], bytes, ins[b], b == 4 ? (size_t)g.BH * g.N * 4 : bytes))
                return fail(REHYAT_EINVAL, "gradients must not overlap the inputs");
        if (out_f32 && overlaps(outs[a], bytes, out_f32, (size_t)g.BH * g.N * g.d * 4))
            return fail(REHYAT_EINVAL, "gradients must not overlap the inputs");
        for (int b = a + 1; b < 3; ++b)
            if (overlaps(outs[a], bytes, outs[b], bytes)) return fail(REHYAT_EINVAL, "gradients must not overlap");
    }
    begin_call();
    hipStream_t s = (hipStream_t)stream;
    const bool bf = g.dtype == REHYAT_BF16;
    const bool bidir = mode == kBidirectional;
    const bool lin = any_linear(g, mode);
    const BwdWorkspace w = bwd_workspace(g, mode);
    ArenaLease lease;
    if ((st = arena_acquire(w.total, s, lease)) != REHYAT_OK) return st;
    char* ws = lease.ptr;

    BwdParams bp{};
    bp.q = q; bp.k = k; bp.v = v; bp.dy = dout; bp.out = out; bp.out_f32 = bf ? out_f32 : nullptr;
    bp.lse = lse; bp.dsum = (const float*)(ws + w.dsum_off);
    bp.dq = dq; bp.dk = dk; bp.dv = dv;
    bp.bh_stride = g.N * g.d;
    bp.N = (int)g.N; bp.HW = g.HW; bp.F = g.F; bp.Tc = g.Tc; bp.To = g.To; bp.C = g.C; bp.BH = g.BH;
    bp.d = g.d; bp.phi = lin ? g.phi : REHYAT_PHI_NONE; bp.lin = lin ? 1 : 0; bp.mode = mode;
    hipError_t e = hip_step([&] { return launch_bwd_dsum(bp, (float*)(ws + w.dsum_off), bf, s); });
    if (e != hipSuccess) return hip_fail(e, "backward dsum launch");
    if (lin) {
        // the forward's states S_t, z_t (both layouts of S_t)
        StateParams sp{};
        sp.k = k; sp.v = v; sp.bh_stride = g.N * g.d;
        sp.HW = g.HW; sp.Tc = g.Tc; sp.To = g.To;
        sp.n_blocks = w.U; sp.sub_rows = w.split.sub_rows; sp.n_sub = w.split.n_sub;
        sp.BH = g.BH; sp.d = g.d; sp.phi = g.phi; sp.mode = mode; sp.F = g.F;
        sp.partial = (float*)(ws + w.part_off);
        sp.items_per_bh = state_items_per_bh(sp);
        e = hip_step([&] { return bf ? launch_state_bf16(sp, s) : launch_state_f32(sp, s); });
        if (e != hipSuccess) return hip_fail(e, "block-state launch");
        ScanParams cp{};
        cp.partial = sp.partial; cp.part = state_part(sp);
        cp.s_hi = ws + w.shi_off; cp.s_lo = ws + w.slo_off; cp.t_hi = ws + w.thi_off; cp.t_lo = ws + w.tlo_off;
        cp.z = (float*)(ws + w.z_off);
        cp.s_chunk_stride = (long long)g.d * g.Dp; cp.s_bh_stride = (long long)g.C * g.d * g.Dp;
        cp.z_chunk_stride = g.Dp; cp.z_bh_stride = (long long)g.C * g.Dp;
        cp.U = w.U; cp.n_sub = w.split.n_sub; cp.BH = g.BH; cp.d = g.d; cp.Dp = g.Dp;
        cp.t_first = bidir ? 0 : 1; cp.t_offset = 0; cp.f32_prep = !bf; cp.mode = mode; cp.C = g.C;
        cp.q = g.To / g.Tc; cp.suffix = bidir ? (float*)(ws + w.suffix_off) : nullptr;
        if ((e = hip_step([&] { return launch_scan(cp, s); })) != hipSuccess) return hip_fail(e, "scan launch");
        // gradient sums per chunk (rows: the chunk's queries, second operand dy)
        StateParams gp = sp;
        gp.k = q; gp.v = dout; gp.mode = bidir ? kChunkRowsAll : kChunkRows;
        gp.n_blocks = w.GU; gp.sub_rows = w.gsplit.sub_rows; gp.n_sub = w.gsplit.n_sub;
        gp.row_lse = lse; gp.row_d = bp.dsum;
        gp.partial = (float*)(ws + w.gpart_off);
        gp.items_per_bh = state_items_per_bh(gp);
        e = hip_step([&] { return bf ? launch_state_bf16(gp, s) : launch_state_f32(gp, s); });
        if (e != hipSuccess) return hip_fail(e, "gradient-state launch");
        ScanParams gc = cp;
        gc.partial = gp.partial; gc.part = state_part(gp); gc.U = w.GU; gc.n_sub = w.gsplit.n_sub;
        gc.s_hi = ws + w.ghi_off; gc.s_lo = ws + w.glo_off; gc.t_hi = ws + w.gthi_off; gc.t_lo = ws + w.gtlo_off;
        gc.z = (float*)(ws + w.gz_off);
        gc.s_bh_stride = (long long)w.gslots * g.d * g.Dp; gc.z_bh_stride = (long long)w.gslots * g.Dp;
        gc.t_first = 0; gc.mode = bidir ? kBidirGrad : kChunkRows;
        gc.suffix = bidir ? (float*)(ws + w.gsuffix_off) : nullptr;
        if ((e = hip_step([&] { return launch_scan(gc, s); })) != hipSuccess) return hip_fail(e, "gradient scan launch");
        bp.st_hi = ws + w.thi_off; bp.st_lo = ws + w.tlo_off; bp.z = (const float*)(ws + w.z_off);
        bp.g_hi = ws + w.ghi_off; bp.g_lo = ws + w.glo_off;
        bp.gt_hi = ws + w.gthi_off; bp.gt_lo = ws + w.gtlo_off; bp.gz = (const float*)(ws + w.gz_off);
        bp.s_stride = (long long)g.d * g.Dp; bp.z_stride = g.Dp;
    }
    if (bf) {
        // dq's work items have the local kernel's shape (the windows of chunk 0
        // are shorter): the same simulated choice of dispatch order
        int tpc = 0, bn = 0;
        dq_launch_shape(bp, tpc, bn);
        LocalParams lp{};
        lp.BH = bp.BH; lp.n_chunks = bp.C; lp.tiles_per_chunk = tpc;
        lp.F = bp.F; lp.Tc = bp.Tc; lp.To = bp.To; lp.HW = bp.HW;
        bp.dq_lpt = choose_lpt_order(lp, bp.BH * bp.C * tpc, bn);
    }
    e = hip_step([&] { return bf ? launch_bwd_bf16(bp, s) : launch_bwd_f32(bp, s); });
    if (e != hipSuccess) return hip_fail(e, "backward launch");
    return REHYAT_OK;
}

// ---------------------------------------------------------------- streaming state
struct StepLayout {
    size_t S_off, shi_off, slo_off, z_off, kp_off[2], vp_off[2], partial_off, total;
    size_t fq_off, fk_off, fkp_off[2];  // learned map: phi rows of the chunk and of the overlap frames
    int n_sub;
    size_t prev_bytes;  // one K (or V) slot
};

StepLayout step_layout(const Geometry& g) {
    StepLayout L{};
    const size_t E = (size_t)g.E;
    // sized for the largest fold (T_c frames); a step never splits into more
    L.n_sub = state_split(g.dtype, (long long)g.Tc * g.HW).n_sub;
    size_t off = 0;
    L.S_off = off; off += align256((size_t)g.BH * E * 4);
    const size_t sprep = (size_t)g.BH * g.d * g.Dp * (g.dtype == REHYAT_BF16 ? 2 : 4);
    L.shi_off = off; off += align256(sprep);
    L.slo_off = off; off += g.dtype == REHYAT_BF16 ? align256(sprep) : 0;
    L.z_off = off; off += align256((size_t)g.BH * g.Dp * 4);
    L.prev_bytes = (size_t)g.BH * g.To * g.HW * g.d * g.elem;
    for (int i = 0; i < 2; ++i) {
        L.kp_off[i] = off; off += align256(L.prev_bytes);
        L.vp_off[i] = off; off += align256(L.prev_bytes);
    }
    L.partial_off = off; off += align256((size_t)g.BH * L.n_sub * E * 4);
    if (g.phi == REHYAT_PHI_MLP2) {
        const size_t chunk_feat = (size_t)g.BH * g.Tc * g.HW * g.Dp * g.elem;
        const size_t prev_feat = (size_t)g.BH * g.To * g.HW * g.Dp * g.elem;
        L.fq_off = off; off += align256(chunk_feat);
        L.fk_off = off; off += align256(chunk_feat);
        for (int i = 0; i < 2; ++i) {
            L.fkp_off[i] = off;
            off += align256(prev_feat);
        }
    }
    L.total = off > 256 ? off : 256;  // never 0: 0 means "invalid arguments"
    return L;
}

// ---------------------------------------------------------------- attention blocks
// The attention part of a DiT block, T_l(x) = f_l(A_l(x) + x) (ReHyAt §3.1,
// first display equation): x [B][N][C] token-major bf16, C = H d;
// A(x) = concat_heads(attn(x Wq^T + bq, (x Wk^T + bk)/sqrt(d), x Wv^T + bv)) Wo^T + bo.
// attn is the hybrid attention (hybrid != 0, the given chunk geometry and
// feature map) or full bidirectional softmax attention (hybrid == 0: one chunk
// over the clip, no linear branch -- the block as it was before conversion).
struct BlockGeometry {
    Geometry attn;  // the attention call's geometry (dense: T_c = F, T_o = 0, no phi)
    int mode;
    long long T;    // tokens B N
    int C;
    size_t act_bytes, q_off, k_off, v_off, y_off, attn_off, attn_bytes;
};

rehyat_status check_block(BlockGeometry& bg, int B, int frames, int tpf, int heads, int d, int hybrid, int Tc, int To,
                          int phi) {
    Geometry g{};
    rehyat_status st = hybrid ? check_common(g, B, heads, frames, tpf, d, Tc, To, phi, REHYAT_BF16)
                              : check_common(g, B, heads, frames, tpf, d, frames, 0, REHYAT_PHI_NONE, REHYAT_BF16);
    if (st != REHYAT_OK) return st;
    const int C = heads * d;
    if (!proj_shape_ok(C, 3 * C, d) || !proj_shape_ok(C, C, d))
        return fail(REHYAT_EUNSUPPORTED, "block width heads*head_dim = %d must be a multiple of 128", C);
    const long long T = (long long)B * g.N;
    if (T * C * 2 >= (1LL << 31))
        return fail(REHYAT_EUNSUPPORTED, "block activations of %lld bytes exceed the 2^31-byte extent the projections "
                    "address", T * C * 2);
    bg.attn = g;
    bg.mode = kCausal;
    bg.T = T;
    bg.C = C;
    bg.act_bytes = (size_t)T * C * 2;
    const size_t a = align256(bg.act_bytes);
    bg.q_off = 0;
    bg.k_off = a;
    bg.v_off = 2 * a;
    bg.y_off = 3 * a;
    bg.attn_off = 4 * a;
    bg.attn_bytes = fwd_workspace_bytes(g, kCausal);
    return REHYAT_OK;
}

rehyat_status check_block_weights(const rehyat_block_weights* w) {
    if (!w) return fail(REHYAT_EINVAL, "null block weights");
    if (!w->w_qkv || !w->b_qkv || !w->w_o || !w->b_o) return fail(REHYAT_EINVAL, "null block weight pointer");
    if (!aligned16(w->w_qkv) || !aligned16(w->b_qkv) || !aligned16(w->w_o) || !aligned16(w->b_o))
        return fail(REHYAT_EINVAL, "block weights must be 16-byte aligned");
    return REHYAT_OK;
}

// One block's launches: x -> out through q, k, v, y in the workspace `ws`.
rehyat_status run_block(const void* x, void* out, const rehyat_block_weights& w, const BlockGeometry& bg, char* ws,
                        hipStream_t s) {
    const Geometry& g = bg.attn;
    ProjParams pq{};
    pq.mode = kProjQKV;
    pq.x = x; pq.w = w.w_qkv; pq.bias = w.b_qkv;
    pq.q = ws + bg.q_off; pq.k = ws + bg.k_off; pq.v = ws + bg.v_off;
    pq.k_scale = 1.0f / std::sqrt((float)g.d);
    pq.T = (int)bg.T; pq.N = (int)g.N; pq.H = g.H; pq.d = g.d; pq.c_in = bg.C; pq.n_out = 3 * bg.C;
    hipError_t e = hip_step([&] { return launch_proj_bf16(pq, s); });
    if (e != hipSuccess) return hip_fail(e, "qkv projection launch");
    rehyat_status st = run_fwd_ws(ws + bg.q_off, ws + bg.k_off, ws + bg.v_off, ws + bg.y_off, g, bg.mode, nullptr,
                                  nullptr, nullptr, nullptr, nullptr, s, nullptr, nullptr, nullptr, nullptr,
                                  bg.attn_bytes ? ws + bg.attn_off : nullptr);
    if (st != REHYAT_OK) return st;
    ProjParams po{};
    po.mode = kProjOut;
    po.x = ws + bg.y_off; po.x_bytes = (int)bg.act_bytes; po.w = w.w_o; po.bias = w.b_o;
    po.resid = x; po.out = out;
    po.T = (int)bg.T; po.N = (int)g.N; po.H = g.H; po.d = g.d; po.c_in = bg.C; po.n_out = bg.C;
    e = hip_step([&] { return launch_proj_bf16(po, s); });
    if (e != hipSuccess) return hip_fail(e, "output projection launch");
    return REHYAT_OK;
}

// A stack of n blocks, x_{l+1} = x_l + A_l(x_l) (f_l taken as the identity:
// the rest of the DiT block is not part of the attention).  Activations
// alternate between two workspace buffers; the last block writes `out`.
rehyat_status stack_entry(const void* x, void* out, const rehyat_block_weights* w, const int* hybrid, int n_blocks,
                          int B, int frames, int tpf, int heads, int d, int Tc, int To, int phi, void* stream) {
    if (n_blocks < 1) return fail(REHYAT_EINVAL, "n_blocks must be >= 1 (got %d)", n_blocks);
    if (!w || !hybrid) return fail(REHYAT_EINVAL, "null weights or hybrid flags");
    if (phi == REHYAT_PHI_MLP2) return fail(REHYAT_EUNSUPPORTED, "the blocks take NONE, ELU1 or POLY2 feature maps");
    BlockGeometry bh{}, bd{};
    bool any_h = false, any_d = false;
    for (int l = 0; l < n_blocks; ++l) (hybrid[l] ? any_h : any_d) = true;
    rehyat_status st;
    if (any_h && (st = check_block(bh, B, frames, tpf, heads, d, 1, Tc, To, phi)) != REHYAT_OK) return st;
    if ((any_d || !any_h) && (st = check_block(bd, B, frames, tpf, heads, d, 0, Tc, To, phi)) != REHYAT_OK) return st;
    for (int l = 0; l < n_blocks; ++l)
        if ((st = check_block_weights(&w[l])) != REHYAT_OK) return st;
    if (!x || !out) return fail(REHYAT_EINVAL, "null tensor pointer");
    if (!aligned16(x) || !aligned16(out)) return fail(REHYAT_EINVAL, "tensor pointers must be 16-byte aligned");
    const BlockGeometry& b0 = any_h ? bh : bd;
    if (overlaps(x, b0.act_bytes, out, b0.act_bytes)) return fail(REHYAT_EINVAL, "out must not overlap x");
    begin_call();
    hipStream_t s = (hipStream_t)stream;
    const size_t a = align256(b0.act_bytes);
    const size_t attn = std::max(any_h ? bh.attn_bytes : 0, any_d ? bd.attn_bytes : 0);
    const size_t per_block = 4 * a + align256(attn);
    const size_t total = per_block + (n_blocks > 1 ? 2 * a : 0);
    ArenaLease lease;
    if ((st = arena_acquire(total, s, lease)) != REHYAT_OK) return st;
    char* ws = lease.ptr;
    const void* cur = x;
    for (int l = 0; l < n_blocks; ++l) {
        void* dst = l == n_blocks - 1 ? out : ws + per_block + (size_t)(l & 1) * a;
        st = run_block(cur, dst, w[l], hybrid[l] ? bh : bd, ws, s);
        if (st != REHYAT_OK) return st;
        cur = dst;
    }
    return REHYAT_OK;
}

}  // namespace

namespace rehyat {

rehyat_status fwd_fixed_workspace(const void* q, const void* k, const void* v, void* out, int B, int H,
                                  int frames, int tokens_per_frame, int head_dim, int chunk_frames,
                                  int overlap_frames, int feature_map, void* stream, fixed_workspace_fn get_ws,
                                  size_t ws_bytes) {
    if (!get_ws) return fail(REHYAT_EINVAL, "internal: no fixed workspace");
    return fwd_entry(q, k, v, out, B, H, frames, tokens_per_frame, head_dim, chunk_frames, overlap_frames,
                     feature_map, REHYAT_BF16, kCausal, stream, nullptr, nullptr, get_ws, ws_bytes);
}

rehyat_status report_hip_error(int err, const char* what) { return hip_fail((hipError_t)err, what); }

}  // namespace rehyat

extern "C" {

rehyat_status rehyat_attn_fwd(const void* q, const void* k, const void* v, void* out, int B, int H,
                              int frames, int tokens_per_frame, int head_dim, int chunk_frames,
                              int overlap_frames, int feature_map, void* stream) {
    return fwd_entry(q, k, v, out, B, H, frames, tokens_per_frame, head_dim, chunk_frames,
                     overlap_frames, feature_map, REHYAT_BF16, kCausal, stream);
}

rehyat_status rehyat_attn_fwd_f32(const void* q, const void* k, const void* v, void* out, int B,
                                  int H, int frames, int tokens_per_frame, int head_dim,
                                  int chunk_frames, int overlap_frames, int feature_map,
                                  void* stream) {
    return fwd_entry(q, k, v, out, B, H, frames, tokens_per_frame, head_dim, chunk_frames,
                     overlap_frames, feature_map, REHYAT_F32, kCausal, stream);
}

rehyat_status rehyat_attn_fwd_bidir(const void* q, const void* k, const void* v, void* out, int B, int H,
                                    int frames, int tokens_per_frame, int head_dim, int chunk_frames,
                                    int overlap_frames, int feature_map, void* stream) {
    return fwd_entry(q, k, v, out, B, H, frames, tokens_per_frame, head_dim, chunk_frames,
                     overlap_frames, feature_map, REHYAT_BF16, kBidirectional, stream);
}

rehyat_status rehyat_attn_fwd_bidir_f32(const void* q, const void* k, const void* v, void* out, int B,
                                        int H, int frames, int tokens_per_frame, int head_dim,
                                        int chunk_frames, int overlap_frames, int feature_map,
                                        void* stream) {
    return fwd_entry(q, k, v, out, B, H, frames, tokens_per_frame, head_dim, chunk_frames,
                     overlap_frames, feature_map, REHYAT_F32, kBidirectional, stream);
}

rehyat_status rehyat_attn_fwd_partials(const void* q, const void* k, const void* v, int dtype,
                                       float* m, float* nt, float* o_s, float* o_l, float* n_l,
                                       int B, int H, int frames, int tokens_per_frame,
                                       int head_dim, int chunk_frames, int overlap_frames,
                                       int feature_map, void* stream) {
    return partials_entry(q, k, v, dtype, m, nt, o_s, o_l, n_l, B, H, frames, tokens_per_frame, head_dim,
                          chunk_frames, overlap_frames, feature_map, kCausal, stream);
}

rehyat_status rehyat_attn_fwd_bidir_partials(const void* q, const void* k, const void* v, int dtype,
                                             float* m, float* nt, float* o_s, float* o_l, float* n_l,
                                             int B, int H, int frames, int tokens_per_frame,
                                             int head_dim, int chunk_frames, int overlap_frames,
                                             int feature_map, void* stream) {
    return partials_entry(q, k, v, dtype, m, nt, o_s, o_l, n_l, B, H, frames, tokens_per_frame, head_dim,
                          chunk_frames, overlap_frames, feature_map, kBidirectional, stream);
}

size_t rehyat_step_state_bytes(int B, int H, int tokens_per_frame, int head_dim, int chunk_frames,
                               int overlap_frames, int feature_map, int dtype) {
    Geometry g{};
    if (check_common(g, B, H, chunk_frames, tokens_per_frame, head_dim, chunk_frames, overlap_frames,
                     feature_map, dtype, feature_map == REHYAT_PHI_MLP2) != REHYAT_OK)
        return 0;
    return step_layout(g).total;
}

rehyat_status rehyat_step_state_init(rehyat_step_state* st, void* buf, size_t bytes, int B, int H,
                                     int tokens_per_frame, int head_dim, int chunk_frames,
                                     int overlap_frames, int feature_map, int dtype) {
    if (!st) return fail(REHYAT_EINVAL, "null state");
    Geometry g{};
    rehyat_status s = check_common(g, B, H, chunk_frames, tokens_per_frame, head_dim, chunk_frames,
                                   overlap_frames, feature_map, dtype, feature_map == REHYAT_PHI_MLP2);
    if (s != REHYAT_OK) return s;
    const size_t need = step_layout(g).total;
    if (!buf) return fail(REHYAT_EINVAL, "null state buffer");
    if (!aligned16(buf)) return fail(REHYAT_EINVAL, "state buffer must be 16-byte aligned");
    if (bytes < need) return fail(REHYAT_EINVAL, "state buffer too small: %zu < %zu bytes", bytes, need);
    std::memset(st, 0, sizeof(*st));
    st->buf = buf;
    st->bytes = bytes;
    st->B = B; st->H = H; st->tokens_per_frame = tokens_per_frame; st->head_dim = head_dim;
    st->chunk_frames = chunk_frames; st->overlap_frames = overlap_frames;
    st->feature_map = feature_map; st->dtype = dtype;
    begin_call();
    return REHYAT_OK;
}

static rehyat_status step_impl(rehyat_step_state* st, const void* q, const void* k, const void* v, void* out,
                               int frames, void* stream, const rehyat_mlp_weights* wq,
                               const rehyat_mlp_weights* wk) {
    if (!st || !st->buf) return fail(REHYAT_EINVAL, "state not initialised");
    Geometry g{};
    const bool mlp = wq != nullptr;
    if (mlp && st->feature_map != REHYAT_PHI_MLP2)
        return fail(REHYAT_EINVAL, "the state was not initialised for REHYAT_PHI_MLP2");
    rehyat_status s0 = check_common(g, st->B, st->H, st->chunk_frames, st->tokens_per_frame,
                                    st->head_dim, st->chunk_frames, st->overlap_frames,
                                    st->feature_map, st->dtype, mlp);
    if (s0 != REHYAT_OK) return s0;
    if (mlp && (s0 = check_mlp(wq, wk)) != REHYAT_OK) return s0;
    const StepLayout L = step_layout(g);
    if (st->bytes < L.total) return fail(REHYAT_EINVAL, "state buffer too small");
    if (frames < 1 || frames > st->chunk_frames)
        return fail(REHYAT_EINVAL, "frames must be in [1, chunk_frames=%d] (got %d)", st->chunk_frames, frames);
    if (st->frames_done % st->chunk_frames != 0)
        return fail(REHYAT_EINVAL, "the stream already ended with a partial chunk");
    if (st->prev_frames < 0 || st->prev_frames > st->overlap_frames || (st->prev_slot & ~1))
        return fail(REHYAT_EINVAL, "corrupt state header");
    if (!q || !k || !v || !out) return fail(REHYAT_EINVAL, "null tensor pointer");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(REHYAT_EINVAL, "tensor pointers must be 16-byte aligned");
    const long long n = (long long)frames * g.HW;
    const size_t bytes = (size_t)g.BH * n * g.d * g.elem;
    if (overlaps(out, bytes, q, bytes) || overlaps(out, bytes, k, bytes) || overlaps(out, bytes, v, bytes) ||
        overlaps(out, bytes, st->buf, st->bytes))
        return fail(REHYAT_EINVAL, "out must not overlap q, k, v or the state buffer");
    begin_call();
    hipStream_t s = (hipStream_t)stream;
    char* base = (char*)st->buf;
    const int P = st->prev_frames * g.HW;
    const int cur = st->prev_slot;
    const long long done = st->frames_done + frames;
    const int keep_frames = (int)std::min<long long>(g.To, done);
    const int keep_rows = keep_frames * g.HW;
    const int evict_rows = P + (int)n - keep_rows;
    const bool fold = g.phi != REHYAT_PHI_NONE && evict_rows > 0;
    const bool copy = keep_rows > 0;
    const SubSplit split = state_split(g.dtype, std::max(evict_rows, 1));
    if (split.n_sub > L.n_sub) return fail(REHYAT_EINVAL, "internal: state split exceeds its buffer");
    if (mlp) {  // phi of the chunk's queries and keys (the overlap frames' phi(k) is carried)
        hipError_t e = hip_step([&] { return launch_mlp(g, wq, wk, q, base + L.fq_off, n, 0, (int)n, k, base + L.fk_off, n, 0, (int)n, s); });
        if (e != hipSuccess) return hip_fail(e, "feature-map launch");
    }

    // the side stream forks here (after the inputs and the chunk's features)
    SideLease side;
    hipStream_t a = s;
    if (fold) {
        rehyat_status ss = side_acquire(s, side);
        if (ss != REHYAT_OK) return ss;
        a = side.side->s;
        hipError_t e = hip_step([&] { return hipEventRecord(side.side->fork, s); });
        if (e != hipSuccess) return hip_fail(e, "fork event");
    }
    bool forked = false;
    // after the side stream waited for the fork, a failure still joins it back,
    // so that nothing the call queued outlives it unordered
    auto failed = [&](hipError_t e, const char* what) {
        if (forked) {
            if (hipEventRecord(side.side->join, a) != hipSuccess || hipStreamWaitEvent(s, side.side->join, 0) != hipSuccess)
                (void)hipStreamSynchronize(a);
        }
        return hip_fail(e, what);
    };

    // 1. local softmax over [prev | chunk] + linear branch from the carried state
    LocalParams lp{};
    lp.q = q; lp.out = out; lp.k = k; lp.v = v;
    lp.kp = P > 0 ? base + L.kp_off[cur] : nullptr;
    lp.vp = P > 0 ? base + L.vp_off[cur] : nullptr;
    lp.bh_stride = n * g.d;
    lp.prev_bh_stride = (long long)g.To * g.HW * g.d;
    lp.prev_rows = P;
    lp.HW = g.HW; lp.F = frames; lp.Tc = frames; lp.To = 0;
    lp.n_chunks = 1; lp.BH = g.BH; lp.d = g.d;
    const int bm = g.dtype == REHYAT_BF16 ? local_bf16_tile_rows(g.d) : local_f32_tile_rows(g.d);
    lp.tiles_per_chunk = (int)((n + bm - 1) / bm);
    lp.phi = g.phi;
    lp.lin_always = (g.phi != REHYAT_PHI_NONE && st->state_nonempty) ? 1 : 0;
    if (!lp.lin_always) lp.phi = REHYAT_PHI_NONE;
    lp.s_hi = base + L.shi_off; lp.s_lo = base + L.slo_off; lp.z = (const float*)(base + L.z_off);
    lp.s_chunk_stride = 0; lp.s_bh_stride = (long long)g.d * g.Dp;
    lp.z_chunk_stride = 0; lp.z_bh_stride = g.Dp;
    if (mlp) {
        lp.fq = base + L.fq_off;
        lp.fq_bh_stride = n * g.Dp;
    }
    // queued first, so that its workgroups take the CUs before the side stream's
    hipError_t e = hip_step([&] { return g.dtype == REHYAT_BF16 ? launch_local_bf16(lp, s) : launch_local_f32(lp, s); });
    if (e != hipSuccess) return failed(e, "local-attention launch");
    if (fold) {
        e = hip_step([&] { return hipStreamWaitEvent(a, side.side->fork, 0); });
        if (e != hipSuccess) return failed(e, "side stream wait");
        forked = true;
    }

    // 2. on the side stream: the sums of the rows leaving the window (fold).
    // They share the GPU with this step's local launch, so the fold uses at
    // most one workgroup per CU that launch leaves idle, each taking several
    // sub-blocks in turn: a workgroup sent to a shader engine with no idle CU
    // would wait for the local launch to end.
    // the copy of the last min(T_o, frames so far) frames for the next window
    // (into the other K/V slot: this step's launches read this one)
    PrevCopyParams pc{};
    if (copy) {
        pc.kp = lp.kp; pc.vp = lp.vp; pc.prev_bh_stride = lp.prev_bh_stride; pc.prev_rows = P;
        pc.k = k; pc.v = v; pc.bh_stride = n * g.d; pc.chunk_rows = (int)n;
        pc.kd = base + L.kp_off[cur ^ 1]; pc.vd = base + L.vp_off[cur ^ 1];
        pc.keep_rows = keep_rows; pc.BH = g.BH; pc.d = g.d; pc.elem_bytes = g.elem;
        if (mlp) {
            pc.fkp = P > 0 ? base + L.fkp_off[cur] : nullptr; pc.fk = base + L.fk_off; pc.fkd = base + L.fkp_off[cur ^ 1];
            pc.fprev_bh_stride = (long long)g.To * g.HW * g.Dp; pc.f_bh_stride = n * g.Dp; pc.f_cols = g.Dp;
        }
    }
    bool copied = false;  // done by the fold's workgroups
    StateParams sp{};
    if (fold) {
        sp.k = k; sp.v = v; sp.kp = lp.kp; sp.vp = lp.vp;
        sp.bh_stride = n * g.d; sp.prev_bh_stride = lp.prev_bh_stride; sp.prev_rows = P;
        sp.HW = g.HW; sp.Tc = g.Tc; sp.To = g.To;
        sp.n_blocks = 1; sp.sub_rows = split.sub_rows;
        sp.n_sub = split.n_sub;
        sp.stream_rows = evict_rows;
        sp.BH = g.BH; sp.d = g.d; sp.phi = g.phi;
        sp.mode = kCausal; sp.F = frames;
        sp.partial = (float*)(base + L.partial_off);
        if (mlp) {
            sp.fk = base + L.fk_off; sp.fk_bh_stride = n * g.Dp;
            sp.fkp = P > 0 ? base + L.fkp_off[cur] : nullptr; sp.fkp_bh_stride = (long long)g.To * g.HW * g.Dp;
        }
        sp.items_per_bh = state_items_per_bh(sp);
        const int idle = cus_per_xcd() * 8 - lp.tiles_per_chunk * lp.BH;
        const int items = sp.items_per_bh * g.BH;
        if (idle > 0 && items > idle) sp.wg_items = (items + idle - 1) / idle;
        // those few workgroups finish long before the local launch: they also
        // make the copy (bf16 K and V; the learned map's phi(K) plane stays below)
        if (copy && !mlp && g.dtype == REHYAT_BF16 && sp.wg_items > 1) {
            sp.copy = pc;
            copied = true;
        }
        e = hip_step([&] { return g.dtype == REHYAT_BF16 ? launch_state_bf16(sp, a) : launch_state_f32(sp, a); });
        if (e != hipSuccess) return failed(e, "block-state launch");
        e = hip_step([&] { return hipEventRecord(side.side->join, a); });
        if (e != hipSuccess) return failed(e, "join event");
        e = hip_step([&] { return hipStreamWaitEvent(s, side.side->join, 0); });
        if (e != hipSuccess) {
            (void)hipStreamSynchronize(a);
            return hip_fail(e, "join wait");
        }
        forked = false;
    }
    // 3. after the local launch (which reads the prepared state), on the
    // caller's stream, in one launch: add the fold into (S, z) and prepare it
    // for the next step, and the overlap copy unless the fold made it
    bool nonempty = st->state_nonempty != 0;
    ScanParams cp{};
    if (fold) {
        cp.partial = sp.partial; cp.part = state_part(sp);
        cp.init = nonempty ? (const float*)(base + L.S_off) : nullptr;
        cp.state_out = (float*)(base + L.S_off);
        cp.s_hi = base + L.shi_off; cp.s_lo = base + L.slo_off; cp.z = (float*)(base + L.z_off);
        cp.s_chunk_stride = 0; cp.s_bh_stride = (long long)g.d * g.Dp;
        cp.z_chunk_stride = 0; cp.z_bh_stride = g.Dp;
        cp.U = 1; cp.n_sub = sp.n_sub; cp.BH = g.BH; cp.d = g.d; cp.Dp = g.Dp;
        cp.t_first = 1; cp.t_offset = 1; cp.f32_prep = g.dtype == REHYAT_F32;
        cp.mode = kCausal; cp.C = 1; cp.q = 0; cp.suffix = nullptr;
        nonempty = true;
    }
    const bool copy_here = copy && !copied;
    if (fold || copy_here) {
        e = hip_step([&] { return launch_scan_copy(fold ? &cp : nullptr, copy_here ? &pc : nullptr, s); });
        if (e != hipSuccess) return hip_fail(e, "state update launch");
    }
    st->prev_slot = copy ? cur ^ 1 : cur;
    st->prev_frames = keep_frames;
    st->state_nonempty = nonempty ? 1 : 0;
    st->frames_done = done;
    return REHYAT_OK;
}

rehyat_status rehyat_attn_step(rehyat_step_state* st, const void* q, const void* k, const void* v,
                               void* out, int frames, void* stream) {
    return step_impl(st, q, k, v, out, frames, stream, nullptr, nullptr);
}

rehyat_status rehyat_attn_step_mlp(rehyat_step_state* st, const void* q, const void* k, const void* v,
                                   void* out, int frames, const rehyat_mlp_weights* phi_q,
                                   const rehyat_mlp_weights* phi_k, void* stream) {
    if (!phi_q || !phi_k) return fail(REHYAT_EINVAL, "null feature-map weights");
    return step_impl(st, q, k, v, out, frames, stream, phi_q, phi_k);
}

rehyat_status rehyat_attn_fwd_mlp(const void* q, const void* k, const void* v, void* out, int dtype, int B,
                                  int H, int frames, int tokens_per_frame, int head_dim, int chunk_frames,
                                  int overlap_frames, int causal, const rehyat_mlp_weights* phi_q,
                                  const rehyat_mlp_weights* phi_k, void* stream) {
    if (!phi_q || !phi_k) return fail(REHYAT_EINVAL, "null feature-map weights");
    return fwd_entry(q, k, v, out, B, H, frames, tokens_per_frame, head_dim, chunk_frames, overlap_frames,
                     REHYAT_PHI_MLP2, dtype, causal ? kCausal : kBidirectional, stream, phi_q, phi_k);
}

rehyat_status rehyat_attn_fwd_mlp_partials(const void* q, const void* k, const void* v, int dtype, float* m,
                                           float* nt, float* o_s, float* o_l, float* n_l, int B, int H,
                                           int frames, int tokens_per_frame, int head_dim, int chunk_frames,
                                           int overlap_frames, int causal, const rehyat_mlp_weights* phi_q,
                                           const rehyat_mlp_weights* phi_k, void* stream) {
    if (!phi_q || !phi_k) return fail(REHYAT_EINVAL, "null feature-map weights");
    return partials_entry(q, k, v, dtype, m, nt, o_s, o_l, n_l, B, H, frames, tokens_per_frame, head_dim,
                          chunk_frames, overlap_frames, REHYAT_PHI_MLP2, causal ? kCausal : kBidirectional,
                          stream, phi_q, phi_k);
}

rehyat_status rehyat_attn_fwd_lse(const void* q, const void* k, const void* v, void* out, float* lse,
                                  float* out_f32, int dtype, int B, int H, int frames, int tokens_per_frame,
                                  int head_dim, int chunk_frames, int overlap_frames, int feature_map, int causal,
                                  void* stream) {
    Geometry g{};
    rehyat_status st = check_common(g, B, H, frames, tokens_per_frame, head_dim, chunk_frames, overlap_frames,
                                    feature_map, dtype);
    if (st != REHYAT_OK) return st;
    if (!q || !k || !v || !out || !lse) return fail(REHYAT_EINVAL, "null tensor pointer");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(lse))
        return fail(REHYAT_EINVAL, "tensor pointers must be 16-byte aligned");
    const size_t bytes = (size_t)g.BH * g.N * g.d * g.elem, lbytes = (size_t)g.BH * g.N * 4;
    if (overlaps(out, bytes, q, bytes) || overlaps(out, bytes, k, bytes) || overlaps(out, bytes, v, bytes) ||
        overlaps(lse, lbytes, out, bytes) || overlaps(lse, lbytes, q, bytes) || overlaps(lse, lbytes, k, bytes) ||
        overlaps(lse, lbytes, v, bytes))
        return fail(REHYAT_EINVAL, "out and lse must not overlap q, k, v or each other");
    if (out_f32 && dtype == REHYAT_BF16) {
        const size_t fb = (size_t)g.BH * g.N * g.d * 4;
        if (!aligned16(out_f32)) return fail(REHYAT_EINVAL, "out_f32 must be 16-byte aligned");
        if (overlaps(out_f32, fb, q, bytes) || overlaps(out_f32, fb, k, bytes) || overlaps(out_f32, fb, v, bytes) ||
            overlaps(out_f32, fb, out, bytes) || overlaps(out_f32, fb, lse, lbytes))
            return fail(REHYAT_EINVAL, "out_f32 must not overlap the other tensors");
    }
    begin_call();
    return run_fwd(q, k, v, out, g, causal ? kCausal : kBidirectional, nullptr, nullptr, nullptr, nullptr,
                   nullptr, (hipStream_t)stream, nullptr, nullptr, lse, out_f32);
}

rehyat_status rehyat_attn_bwd(const void* q, const void* k, const void* v, const void* out, const float* out_f32,
                              const float* lse, const void* dout, void* dq, void* dk, void* dv, int dtype, int B,
                              int H, int frames, int tokens_per_frame, int head_dim, int chunk_frames,
                              int overlap_frames, int feature_map, int causal, void* stream) {
    return bwd_entry(q, k, v, out, out_f32, lse, dout, dq, dk, dv, dtype, B, H, frames, tokens_per_frame, head_dim,
                     chunk_frames, overlap_frames, feature_map, causal ? kCausal : kBidirectional, stream);
}

rehyat_status rehyat_block_fwd(const void* x, void* out, const rehyat_block_weights* w, int B, int frames,
                               int tokens_per_frame, int heads, int head_dim, int hybrid, int chunk_frames,
                               int overlap_frames, int feature_map, void* stream) {
    const int flag = hybrid ? 1 : 0;
    return stack_entry(x, out, w, &flag, 1, B, frames, tokens_per_frame, heads, head_dim, chunk_frames,
                       overlap_frames, feature_map, stream);
}

rehyat_status rehyat_stack_fwd(const void* x, void* out, const rehyat_block_weights* w, const int* hybrid,
                               int n_blocks, int B, int frames, int tokens_per_frame, int heads, int head_dim,
                               int chunk_frames, int overlap_frames, int feature_map, void* stream) {
    return stack_entry(x, out, w, hybrid, n_blocks, B, frames, tokens_per_frame, heads, head_dim, chunk_frames,
                       overlap_frames, feature_map, stream);
}

rehyat_status rehyat_feature_mlp(const void* x, void* phi, int dtype, int B, int H, int rows, int head_dim,
                                 const rehyat_mlp_weights* w, void* stream) {
    Geometry g{};
    rehyat_status st = check_common(g, B, H, 1, rows, head_dim, 1, 0, REHYAT_PHI_MLP2, dtype, true);
    if (st != REHYAT_OK) return st;
    if ((st = check_mlp(w, w)) != REHYAT_OK) return st;
    if (!x || !phi) return fail(REHYAT_EINVAL, "null tensor pointer");
    if (!aligned16(x) || !aligned16(phi)) return fail(REHYAT_EINVAL, "tensor pointers must be 16-byte aligned");
    const size_t xb = (size_t)g.BH * rows * head_dim * g.elem, pb = 2 * xb;
    if (overlaps(x, xb, phi, pb)) return fail(REHYAT_EINVAL, "phi must not overlap x");
    begin_call();
    hipError_t e = hip_step([&] { return launch_mlp(g, w, w, x, phi, rows, 0, rows, nullptr, nullptr, 0, 0, 0, (hipStream_t)stream); });
    return e == hipSuccess ? REHYAT_OK : hip_fail(e, "feature-map launch");
}

rehyat_status rehyat_workspace_release(void* stream) {
    begin_call();
    side_release((hipStream_t)stream);
    return arena_release((hipStream_t)stream);
}

void rehyat_debug_inject_hip_error(int step) { g_inject_at = step < 0 ? -1 : step; }

int rehyat_debug_hip_steps(void) { return g_steps; }

rehyat_status rehyat_set_profile_events(void* const* events, int n_events) {
    if (n_events == 0) {
        for (auto& e : g_prof) e = nullptr;
        return REHYAT_OK;
    }
    if (n_events != 4 || !events) return fail(REHYAT_EINVAL, "n_events must be 0 or 4");
    for (int i = 0; i < 4; ++i)
        if (!events[i]) return fail(REHYAT_EINVAL, "null event");
    for (int i = 0; i < 4; ++i) g_prof[i] = (hipEvent_t)events[i];
    return REHYAT_OK;
}

const char* rehyat_status_string(int status) {
    switch (status) {
    case REHYAT_OK: return "ok";
    case REHYAT_EINVAL: return "invalid argument";
    case REHYAT_EUNSUPPORTED: return "unsupported configuration";
    case REHYAT_ENOMEM: return "out of device memory";
    case REHYAT_EHIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

const char* rehyat_last_error(void) { return g_last_error.c_str(); }

const char* rehyat_version(void) { return "librehyat 0.1.0 (gfx950)"; }

}  // extern "C"
