// host_sanitize_check.cpp -- the host side of librehyat (argument validation,
// geometry, workspace sizing, the step-state header, error reporting) built
// for the CPU with AddressSanitizer and UndefinedBehaviorSanitizer and driven
// through every entry point of include/rehyat.h.
//
// The kernel launchers of kernels.h are replaced by stubs that count calls.
// Every call either fails validation or runs with the fault-injection hook
// armed at HIP step 0, so no HIP runtime call is made and no stub is reached:
// the program needs no GPU.  It prints "host sanitize check: N calls, 0
// failures" and exits 0 when every status matches what the contract says.
#include <cstdio>
#include <cstring>

#include "../../include/rehyat.h"
#include "kernels.h"

namespace rehyat {
static int g_launches = 0;
hipError_t launch_local_bf16(const LocalParams&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_local_f32(const LocalParams&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_state_bf16(const StateParams&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_state_f32(const StateParams&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_scan(const ScanParams&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_prev_copy(const PrevCopyParams&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_scan_copy(const ScanParams*, const PrevCopyParams*, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_phi_mlp_bf16(const MlpParams&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_phi_mlp_f32(const MlpParams&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_bwd_dsum(const BwdParams&, float*, bool, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_bwd_bf16(const BwdParams&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_bwd_f32(const BwdParams&, hipStream_t) { ++g_launches; return hipSuccess; }
void dq_launch_shape(const BwdParams&, int& tiles_per_chunk, int& key_tile) { tiles_per_chunk = 1; key_tile = 64; }
hipError_t launch_proj_bf16(const ProjParams&, hipStream_t) { ++g_launches; return hipSuccess; }
bool proj_shape_ok(int c_in, int n_out, int head_dim) {
    return c_in % 32 == 0 && n_out % 128 == 0 && head_dim % 32 == 0 && c_in % head_dim == 0;
}
bool phi_mlp_hidden_ok(int hidden) { return hidden == 32 || hidden == 64 || hidden == 128 || hidden == 256; }
int local_bf16_tile_rows(int) { return 256; }
int local_bf16_key_tile(int) { return 128; }
int local_f32_tile_rows(int) { return 64; }
}  // namespace rehyat

static int g_calls = 0, g_failures = 0;

static void expect(int got, int want, const char* what) {
    ++g_calls;
    if (got != want) {
        ++g_failures;
        std::printf("FAIL %s: status %d, expected %d (%s)\n", what, got, want, rehyat_last_error());
    }
    if (got != REHYAT_OK && std::strlen(rehyat_last_error()) == 0) {
        ++g_failures;
        std::printf("FAIL %s: empty error message\n", what);
    }
}

// aligned fake device addresses: never dereferenced on the host
static void* P(unsigned long i) { return (void*)(0x100000ul * i); }

int main() {
    const int I = REHYAT_EINVAL, U = REHYAT_EUNSUPPORTED, H = REHYAT_EHIP;
    // ---- whole-clip forward: every validation path
    expect(rehyat_attn_fwd(P(1), P(2), P(3), P(4), 0, 1, 4, 8, 64, 1, 1, 1, nullptr), I, "B=0");
    expect(rehyat_attn_fwd(P(1), P(2), P(3), P(4), 1, -3, 4, 8, 64, 1, 1, 1, nullptr), I, "H<0");
    expect(rehyat_attn_fwd(P(1), P(2), P(3), P(4), 1, 1, 0, 8, 64, 1, 1, 1, nullptr), I, "frames=0");
    expect(rehyat_attn_fwd(P(1), P(2), P(3), P(4), 1, 1, 4, 0, 64, 1, 1, 1, nullptr), I, "hw=0");
    expect(rehyat_attn_fwd(P(1), P(2), P(3), P(4), 1, 1, 4, 8, 64, 0, 1, 1, nullptr), I, "Tc=0");
    expect(rehyat_attn_fwd(P(1), P(2), P(3), P(4), 1, 1, 4, 8, 64, 1, -1, 1, nullptr), I, "To<0");
    expect(rehyat_attn_fwd(P(1), P(2), P(3), P(4), 1, 1, 4, 8, 64, 1, 1, 9, nullptr), I, "phi");
    expect(rehyat_attn_fwd(P(1), P(2), P(3), P(4), 1, 1, 4, 8, 64, 1, 1, 3, nullptr), I, "mlp w/o weights");
    expect(rehyat_attn_fwd(P(1), P(2), P(3), P(4), 1, 1, 4, 8, 48, 1, 1, 1, nullptr), U, "d=48");
    expect(rehyat_attn_fwd(P(1), P(2), P(3), P(4), 1, 1, 1 << 20, 1 << 20, 64, 1, 1, 1, nullptr), I, "N>2^30");
    expect(rehyat_attn_fwd(P(1), P(2), P(3), P(4), 1, 1, 8192, 1024, 128, 3, 1, 1, nullptr), U, "extent");
    expect(rehyat_attn_fwd(P(1), P(2), P(3), P(4), 1 << 13, 1 << 12, 4, 8, 64, 1, 1, 1, nullptr), I, "B*H");
    expect(rehyat_attn_fwd(nullptr, P(2), P(3), P(4), 1, 1, 4, 8, 64, 1, 1, 1, nullptr), I, "null q");
    expect(rehyat_attn_fwd(P(1), P(2), P(3), (char*)P(4) + 4, 1, 1, 4, 8, 64, 1, 1, 1, nullptr), I, "misaligned");
    expect(rehyat_attn_fwd(P(1), P(2), P(3), (char*)P(1) + 16, 1, 1, 4, 8, 64, 1, 1, 1, nullptr), I, "overlap");
    expect(rehyat_attn_fwd_f32(P(1), P(2), P(3), P(4), 1, 1, 4, 8, 8, 1, 1, 1, nullptr), U, "f32 d=8");
    expect(rehyat_attn_fwd_bidir(P(1), P(2), P(3), P(4), 1, 1, 4, 8, 64, 1, -2, 1, nullptr), I, "bidir To");
    expect(rehyat_attn_fwd_bidir_f32(P(1), P(2), P(3), P(4), 1, 1, 4, 8, 64, 1, 1, 7, nullptr), I, "bidir phi");
    // ---- partials
    expect(rehyat_attn_fwd_partials(P(1), P(2), P(3), 1, nullptr, nullptr, nullptr, nullptr, nullptr, 1, 1, 4, 8,
                                    64, 1, 1, 1, nullptr), I, "no partials");
    expect(rehyat_attn_fwd_partials(P(1), P(2), P(3), 7, (float*)P(5), nullptr, nullptr, nullptr, nullptr, 1, 1, 4,
                                    8, 64, 1, 1, 1, nullptr), I, "partials dtype");
    expect(rehyat_attn_fwd_bidir_partials(P(1), P(2), P(3), 1, (float*)((char*)P(5) + 8), nullptr, nullptr,
                                          nullptr, nullptr, 1, 1, 4, 8, 64, 1, 1, 1, nullptr), I, "partials align");
    // ---- learned maps
    rehyat_mlp_weights w{P(10), (const float*)P(11), P(12), (const float*)P(13), 256};
    rehyat_mlp_weights bad = w;
    bad.hidden = 96;
    expect(rehyat_attn_fwd_mlp(P(1), P(2), P(3), P(4), 1, 1, 1, 4, 8, 64, 1, 1, 1, nullptr, &w, nullptr), I, "mlp null");
    expect(rehyat_attn_fwd_mlp(P(1), P(2), P(3), P(4), 1, 1, 1, 4, 8, 64, 1, 1, 1, &bad, &w, nullptr), U, "hidden");
    bad = w;
    bad.b1 = nullptr;
    expect(rehyat_attn_fwd_mlp(P(1), P(2), P(3), P(4), 1, 1, 1, 4, 8, 64, 1, 1, 1, &w, &bad, nullptr), I, "b1 null");
    expect(rehyat_feature_mlp(P(1), (char*)P(1) + 64, 1, 1, 1, 8, 64, &w, nullptr), I, "mlp overlap");
    expect(rehyat_attn_fwd_mlp_partials(P(1), P(2), P(3), 1, nullptr, nullptr, nullptr, nullptr, nullptr, 1, 1, 4, 8,
                                        64, 1, 1, 1, &w, &w, nullptr), I, "mlp partials none");
    // ---- training direction
    expect(rehyat_attn_fwd_lse(P(1), P(2), P(3), P(4), nullptr, nullptr, 1, 1, 1, 4, 8, 64, 1, 1, 1, 1, nullptr), I,
           "lse null");
    expect(rehyat_attn_fwd_lse(P(1), P(2), P(3), P(4), (float*)P(4), nullptr, 1, 1, 1, 4, 8, 64, 1, 1, 1, 1, nullptr),
           I, "lse overlap");
    expect(rehyat_attn_bwd(P(1), P(2), P(3), P(4), nullptr, (const float*)P(5), P(6), P(7), P(8), P(1), 1, 1, 1, 4, 8,
                           64, 1, 1, 1, 1, nullptr), I, "bwd dv aliases q");
    expect(rehyat_attn_bwd(P(1), P(2), P(3), P(4), nullptr, (const float*)P(5), P(6), P(7), P(8), nullptr, 1, 1, 1, 4,
                           8, 64, 1, 1, 1, 1, nullptr), I, "bwd null dv");
    // ---- streaming state
    expect((int)(rehyat_step_state_bytes(1, 1, 8, 64, 0, 1, 1, 1) == 0), 1, "state bytes Tc=0");
    const size_t need = rehyat_step_state_bytes(1, 2, 8, 64, 2, 1, 1, 1);
    expect((int)(need > 0), 1, "state bytes");
    rehyat_step_state st;
    std::memset(&st, 0, sizeof st);
    expect(rehyat_step_state_init(&st, P(20), need - 1, 1, 2, 8, 64, 2, 1, 1, 1), I, "state small");
    expect(rehyat_step_state_init(&st, nullptr, need, 1, 2, 8, 64, 2, 1, 1, 1), I, "state null");
    expect(rehyat_step_state_init(nullptr, P(20), need, 1, 2, 8, 64, 2, 1, 1, 1), I, "state ptr null");
    expect(rehyat_step_state_init(&st, P(20), need, 1, 2, 8, 64, 2, 1, 1, 1), REHYAT_OK, "state init");
    expect(rehyat_attn_step(&st, P(1), P(2), P(3), P(4), 3, nullptr), I, "step frames");
    expect(rehyat_attn_step(&st, P(1), P(2), P(3), P(20), 1, nullptr), I, "step out overlaps state");
    st.prev_frames = 5;
    expect(rehyat_attn_step(&st, P(1), P(2), P(3), P(4), 1, nullptr), I, "corrupt header");
    st.prev_frames = 0;
    expect(rehyat_attn_step_mlp(&st, P(1), P(2), P(3), P(4), 1, &w, &w, nullptr), I, "step mlp on elu1 state");
    expect(rehyat_set_profile_events(nullptr, 3), I, "profile events");
    // ---- attention blocks
    rehyat_block_weights bw{P(30), (const float*)P(31), P(32), (const float*)P(33)};
    rehyat_block_weights bwn = bw;
    bwn.b_o = nullptr;
    const int hyb[3] = {1, 0, 1};
    expect(rehyat_block_fwd(P(1), P(2), nullptr, 1, 4, 8, 2, 64, 1, 1, 1, 1, nullptr), I, "block null weights");
    expect(rehyat_block_fwd(P(1), P(2), &bwn, 1, 4, 8, 2, 64, 1, 1, 1, 1, nullptr), I, "block null b_o");
    expect(rehyat_block_fwd(P(1), P(2), &bw, 1, 4, 8, 3, 32, 1, 1, 1, 1, nullptr), U, "block width 96");
    expect(rehyat_block_fwd(P(1), (char*)P(1) + 64, &bw, 1, 4, 8, 2, 64, 1, 1, 1, 1, nullptr), I, "block overlap");
    expect(rehyat_block_fwd(P(1), P(2), &bw, 1, 4, 8, 2, 64, 1, 1, 1, 3, nullptr), U, "block mlp");
    expect(rehyat_stack_fwd(P(1), P(2), &bw, hyb, 0, 1, 4, 8, 2, 64, 1, 1, 1, nullptr), I, "stack n=0");
    expect(rehyat_stack_fwd(P(1), P(2), &bw, nullptr, 1, 1, 4, 8, 2, 64, 1, 1, 1, nullptr), I, "stack null flags");
    expect(rehyat_block_fwd(P(1), P(2), &bw, 1, 1 << 13, 1 << 10, 2, 64, 1, 3, 1, 1, nullptr), U, "block extent");
    // ---- valid calls stopped at their first HIP step by the armed hook
    struct { const char* name; int want; } armed[] = {{"fwd", H}, {"fwd none", H}, {"bidir f32", H}, {"partials", H},
                                                      {"lse", H}, {"bwd", H}, {"step", H}, {"mlp", H},
                                                      {"feature mlp", H}, {"release", H}, {"block", H},
                                                      {"stack", H}};
    for (int i = 0; i < (int)(sizeof armed / sizeof armed[0]); ++i) {
        rehyat_debug_inject_hip_error(0);
        int s = -1;
        switch (i) {
        case 0: s = rehyat_attn_fwd(P(1), P(2), P(3), P(4), 1, 2, 7, 33, 64, 3, 1, 1, nullptr); break;
        case 1: s = rehyat_attn_fwd(P(1), P(2), P(3), P(4), 1, 2, 7, 33, 64, 3, 1, 0, nullptr); break;
        case 2: s = rehyat_attn_fwd_bidir_f32(P(1), P(2), P(3), P(4), 2, 1, 5, 17, 16, 2, 3, 2, nullptr); break;
        case 3:
            s = rehyat_attn_fwd_partials(P(1), P(2), P(3), 1, (float*)P(5), (float*)P(6), (float*)P(7),
                                         (float*)P(8), (float*)P(9), 1, 2, 7, 33, 64, 3, 1, 2, nullptr);
            break;
        case 4: s = rehyat_attn_fwd_lse(P(1), P(2), P(3), P(4), (float*)P(5), (float*)P(6), 1, 1, 2, 7, 33, 128, 3, 1,
                                        1, 0, nullptr); break;
        case 5: s = rehyat_attn_bwd(P(1), P(2), P(3), P(4), nullptr, (const float*)P(5), P(6), P(7), P(8), P(9), 1, 1,
                                    2, 7, 33, 64, 3, 1, 2, 1, nullptr); break;
        case 6: s = rehyat_attn_step(&st, P(1), P(2), P(3), P(4), 2, nullptr); break;
        case 7: s = rehyat_attn_fwd_mlp(P(1), P(2), P(3), P(4), 1, 1, 2, 7, 33, 64, 3, 1, 1, &w, &w, nullptr); break;
        case 8: s = rehyat_feature_mlp(P(1), P(2), 1, 1, 2, 33, 64, &w, nullptr); break;
        case 9: s = rehyat_workspace_release(nullptr); break;
        case 10: s = rehyat_block_fwd(P(1), P(2), &bw, 1, 5, 40, 2, 64, 1, 2, 1, 1, nullptr); break;
        case 11: {
            rehyat_block_weights three[3] = {bw, bw, bw};
            s = rehyat_stack_fwd(P(1), P(3), three, hyb, 3, 1, 5, 40, 2, 64, 2, 1, 2, nullptr);
            break;
        }
        }
        expect(s, armed[i].want, armed[i].name);
        if (!std::strstr(rehyat_last_error(), "injected")) {
            ++g_failures;
            std::printf("FAIL %s: %s\n", armed[i].name, rehyat_last_error());
        }
        if (rehyat_debug_hip_steps() != 1) {
            ++g_failures;
            std::printf("FAIL %s: %d HIP steps\n", armed[i].name, rehyat_debug_hip_steps());
        }
    }
    rehyat_debug_inject_hip_error(-1);
    expect((int)(st.frames_done == 0), 1, "failed step leaves the header");
    // ---- strings
    for (int s = -1; s <= 5; ++s) expect((int)(std::strlen(rehyat_status_string(s)) > 0), 1, "status string");
    expect((int)(std::strncmp(rehyat_version(), "librehyat", 9) == 0), 1, "version");
    if (rehyat::g_launches != 0) {
        ++g_failures;
        std::printf("FAIL: %d kernel launches reached\n", rehyat::g_launches);
    }
    std::printf("host sanitize check: %d calls, %d failures\n", g_calls, g_failures);
    return g_failures == 0 ? 0 : 1;
}
