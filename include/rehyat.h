/*
 * rehyat.h -- C ABI of librehyat, the ReHyAt recurrent hybrid attention forward
 * pass for AMD Instinct MI355X (gfx950).
 *
 * Method: "ReHyAt: Recurrent Hybrid Attention for Video Diffusion Transformers"
 * (Ghafoorian & Habibian, arXiv 2601.04342).  For a query token i of temporal
 * chunk t (T_c frames of HW tokens each, frame-major token order):
 *
 *   softmax set  T^S_t = { j : max(t T_c - T_o, 0) HW <= j < min((t+1) T_c, F) HW }
 *   linear set   T^L_t = { j : j < max(t T_c - T_o, 0) HW }           (§3.3 equation)
 *   keys after the chunk are ignored (the causal, recurrent partition);
 *
 *   a^S = sum_{T^S} exp(q.k) v      n^S = sum_{T^S} exp(q.k)
 *   a^L = sum_{T^L} (phi(q).phi(k)) v   n^L = sum_{T^L} phi(q).phi(k)  (§3.1)
 *   y   = (a^S + a^L) / (n^S + n^L)                          (§3.2, first equation)
 *
 * The linear sums over T^L_t are carried from chunk to chunk as the state
 * (S = sum phi(k) v^T, z = sum phi(k)) of the chunk-wise RNN form, whose memory
 * does not grow with the length of the video (abstract and §3.3).
 *
 * Conventions shared by every entry point
 *   - Tensors are device pointers to contiguous [B][H][N][head_dim] arrays,
 *     N = frames * tokens_per_frame, tokens frame-major.  The caller owns them.
 *   - The softmax similarity is exp(q.k) with no extra scale: callers fold the
 *     usual 1/sqrt(head_dim) into k (or q).
 *   - bf16 entry points: bf16 in and out, fp32 accumulation and fp32 state.
 *     _f32 entry points: fp32 in and out.
 *   - head_dim: 32, 64 or 128 for bf16; 16, 32, 64 or 128 for fp32.
 *     Pointers must be 16-byte aligned.  chunk_frames >= 1, overlap_frames >= 0
 *     (overlap_frames >= chunk_frames is allowed); the last chunk may be partial.
 *   - Calls are asynchronous and ordered on `stream` (a hipStream_t; NULL = the
 *     null stream).  Arguments are validated on the host before any GPU work is
 *     queued; on failure nothing is queued, the status is returned and
 *     rehyat_last_error() describes it.  Errors raised by the HIP runtime while
 *     queueing map to REHYAT_EHIP; the kernels already queued by that call may
 *     then have run, and its outputs are undefined.  No call aborts or throws
 *     across the ABI.
 *   - Streams and threads: the workspace of the whole-clip calls comes from an
 *     arena per (device, stream), so calls on different streams may run
 *     concurrently.  Calls on one stream from several threads are serialised
 *     while they queue their launches (each call holds its arena until its last
 *     launch is queued).  The arena of a stream lives until the process ends or
 *     rehyat_workspace_release() frees it; release it before destroying a stream
 *     that made calls.  A streaming step (rehyat_attn_step*) with a linear
 *     branch queues the sums of the keys leaving its window on a library-owned
 *     side stream of (device, stream), beside its local-attention kernel: the
 *     side stream waits for an event recorded on `stream`, and `stream` waits
 *     for an event recorded on the side stream before the rest of the step.
 *     Work queued on `stream` afterwards is ordered after the whole step, as
 *     for any other call, and graph capture of `stream` takes the side stream
 *     in.  rehyat_workspace_release() destroys that side stream too.
 *   - Graph capture: the calls queue kernel launches and event records and
 *     waits only (no memsets, copies or allocations), once the stream's
 *     workspace (and, for streaming steps, its side stream) exists: make one
 *     eager call on the stream before capturing it, or use
 *     rehyat_attn_fwd_noalloc.  A captured stream of steps replays as that
 *     stream from the state it started from.
 *   - Sizes: the rows of one (b, h) are addressed with 32-bit byte offsets, so
 *     frames * tokens_per_frame * (row bytes) must stay below 2^31, where a row
 *     is head_dim elements (2 head_dim with the learned maps); larger clips are
 *     rejected with REHYAT_EUNSUPPORTED (at head_dim 128 in bf16: 8,388,607 tokens).
 */
#ifndef REHYAT_H
#define REHYAT_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rehyat_feature_map {
    REHYAT_PHI_NONE = 0,  /* no linear branch: softmax over the local window only */
    REHYAT_PHI_ELU1 = 1,  /* phi(x) = elu(x) + 1 (alpha 1), D' = head_dim (§3.1) */
    REHYAT_PHI_POLY2 = 2, /* phi(x) = [elu(x) + 1, x*x], D' = 2 head_dim: a parameter-free
                             degree-2 instance of the polynomial map of §3.2 */
    REHYAT_PHI_MLP2 = 3   /* learned degree-2 map (see rehyat_mlp_weights), D' = 2 head_dim;
                             only through the _mlp entry points, which take its weights */
} rehyat_feature_map;

typedef enum rehyat_status {
    REHYAT_OK = 0,
    REHYAT_EINVAL = 1,        /* invalid argument (null pointer, bad size, misalignment) */
    REHYAT_EUNSUPPORTED = 2,  /* valid but not built (head_dim, dtype, feature map) */
    REHYAT_ENOMEM = 3,        /* device workspace could not be allocated */
    REHYAT_EHIP = 4           /* the HIP runtime reported an error */
} rehyat_status;

typedef enum rehyat_dtype { REHYAT_F32 = 0, REHYAT_BF16 = 1 } rehyat_dtype;

/*
 * Whole-clip forward, parallel chunked form (§3.2-§3.3).
 *   q, k, v : in,  [B][H][frames*tokens_per_frame][head_dim] bf16
 *   out     : out, same shape and dtype; must not alias q, k or v
 * A transient fp32 workspace (about ceil(F/T_c) * B * H * (D' head_dim + D') * 12 bytes)
 * comes from the arena of (current device, stream), which the library grows on
 * demand and keeps until the process ends or rehyat_workspace_release()
 * (REHYAT_ENOMEM if it cannot grow).  With
 * chunk_frames >= frames and REHYAT_PHI_NONE this is plain bidirectional
 * softmax attention (the dense comparison point).
 */
rehyat_status rehyat_attn_fwd(const void* q, const void* k, const void* v, void* out,
                              int B, int H, int frames, int tokens_per_frame, int head_dim,
                              int chunk_frames, int overlap_frames, int feature_map,
                              void* stream);

/*
 * Allocation-free rehyat_attn_fwd, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments, validation, kernels and results as
 * rehyat_attn_fwd, but the workspace is a fixed file-scope device array of
 * rehyat_noalloc_workspace_limit() bytes (64 MiB) on each device, held by the
 * library until the process ends; no hipMalloc or hipFree is called.  A call
 * that needs more workspace returns REHYAT_ENOMEM (a 21-frame clip of
 * 1560-token frames with 12 heads of 128 needs about 20 MB with elu+1, about
 * 40 MB with POLY2 or as a B = 2 pair).  Every call on a device shares the
 * array: calls that overlap on one device (several streams or threads) race,
 * so the caller must serialise them.
 */
rehyat_status rehyat_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out,
                                      int B, int H, int frames, int tokens_per_frame, int head_dim,
                                      int chunk_frames, int overlap_frames, int feature_map,
                                      void* stream);
/* Bytes of the fixed workspace of rehyat_attn_fwd_noalloc. */
size_t rehyat_noalloc_workspace_limit(void);

/* Same contract with fp32 q, k, v, out. */
rehyat_status rehyat_attn_fwd_f32(const void* q, const void* k, const void* v, void* out,
                                  int B, int H, int frames, int tokens_per_frame, int head_dim,
                                  int chunk_frames, int overlap_frames, int feature_map,
                                  void* stream);

/*
 * Forward that writes per-query partials instead of `out` (a verification aid:
 * it lets each branch be checked on its own).  Same kernels as rehyat_attn_fwd.
 * dtype selects bf16 or fp32 inputs.  Outputs are caller-owned fp32 device
 * arrays; each may be NULL:
 *   m   [B][H][N]     max of q.k over the softmax set
 *   nt  [B][H][N]     sum over the softmax set of exp(q.k - m)
 *   o_s [B][H][N][d]  softmax-branch output a^S / n^S
 *   o_l [B][H][N][d]  linear-branch output a^L / n^L (0 where n^L = 0)
 *   n_l [B][H][N]     n^L
 */
rehyat_status rehyat_attn_fwd_partials(const void* q, const void* k, const void* v, int dtype,
                                       float* m, float* nt, float* o_s, float* o_l, float* n_l,
                                       int B, int H, int frames, int tokens_per_frame,
                                       int head_dim, int chunk_frames, int overlap_frames,
                                       int feature_map, void* stream);

/*
 * Bidirectional (non-causal) form, ReHyAt §3.2 with overlap (second partition
 * equation): the softmax set of chunk t is the same window as above, and the
 * linear set is every other key of the clip -- the keys before the window and
 * the keys of every later chunk.  Same arguments, layouts, ownership, errors
 * and stream behaviour as rehyat_attn_fwd / rehyat_attn_fwd_f32.  The linear
 * state of chunk t is formed as a prefix plus a suffix of block sums (two
 * separate fp32 sums, never a total minus the window).  There is no streaming
 * form: a chunk's output depends on later chunks.
 */
rehyat_status rehyat_attn_fwd_bidir(const void* q, const void* k, const void* v, void* out,
                                    int B, int H, int frames, int tokens_per_frame, int head_dim,
                                    int chunk_frames, int overlap_frames, int feature_map,
                                    void* stream);
rehyat_status rehyat_attn_fwd_bidir_f32(const void* q, const void* k, const void* v, void* out,
                                        int B, int H, int frames, int tokens_per_frame, int head_dim,
                                        int chunk_frames, int overlap_frames, int feature_map,
                                        void* stream);
/* Per-query partials of the bidirectional form (see rehyat_attn_fwd_partials). */
rehyat_status rehyat_attn_fwd_bidir_partials(const void* q, const void* k, const void* v, int dtype,
                                             float* m, float* nt, float* o_s, float* o_l, float* n_l,
                                             int B, int H, int frames, int tokens_per_frame,
                                             int head_dim, int chunk_frames, int overlap_frames,
                                             int feature_map, void* stream);

/*
 * Streaming (chunk-wise RNN) form, §3.3: one call per chunk of frames, with
 * memory that does not depend on how many frames have been processed.
 *
 * The state lives in one caller-owned device buffer of
 * rehyat_step_state_bytes() bytes plus this host struct.  It holds the fp32
 * linear state (S, z) of every key that has left the softmax window, the keys
 * and values of the last min(overlap_frames, frames so far) frames, and a
 * small fp32 workspace.  Its contents need no initialisation: a freshly
 * initialised state (frames_done == 0) never reads them.  Saving the buffer
 * and the struct and restoring both resumes the stream exactly.
 */
typedef struct rehyat_step_state {
    void* buf;              /* device buffer, caller-owned */
    size_t bytes;           /* its size */
    int B, H, tokens_per_frame, head_dim, chunk_frames, overlap_frames, feature_map, dtype;
    int prev_frames;        /* frames of K/V held for the next window (library-maintained) */
    int prev_slot;          /* which of the two K/V slots holds them (library-maintained) */
    int state_nonempty;     /* (S, z) has absorbed at least one key (library-maintained) */
    long long frames_done;  /* frames processed so far (library-maintained) */
} rehyat_step_state;

/* Bytes of device buffer the state needs; 0 if the arguments are invalid. */
size_t rehyat_step_state_bytes(int B, int H, int tokens_per_frame, int head_dim,
                               int chunk_frames, int overlap_frames, int feature_map, int dtype);

/* Validate the geometry and bind `buf` (at least rehyat_step_state_bytes()).
 * Host only: queues no GPU work. */
rehyat_status rehyat_step_state_init(rehyat_step_state* st, void* buf, size_t bytes, int B, int H,
                                     int tokens_per_frame, int head_dim, int chunk_frames,
                                     int overlap_frames, int feature_map, int dtype);

/*
 * Attend one chunk: q, k, v, out are [B][H][frames*tokens_per_frame][head_dim]
 * in the state's dtype, 1 <= frames <= chunk_frames.  Every call but the last
 * of a stream must pass frames == chunk_frames; then the concatenated outputs
 * equal rehyat_attn_fwd on the concatenated inputs.  Updates `st`.
 * Concurrent calls on one state are not allowed.  A step that returns
 * REHYAT_EHIP leaves the host header unchanged, but the device buffer may
 * already hold part of the chunk's update: restore a saved state (buffer and
 * header) before continuing the stream.
 */
rehyat_status rehyat_attn_step(rehyat_step_state* st, const void* q, const void* k, const void* v,
                               void* out, int frames, void* stream);

/*
 * Learned feature maps (ReHyAt §3.2, the polynomial map phi(x) = [psi_1(x),
 * psi_2(x)^2] after the partition equations; §4.3 "Model Hyperparameters" and
 * appendix §7.1: psi is a two-layer MLP of degree 2, with separate maps for
 * queries and keys).  Per head h and row x (head_dim values):
 *
 *   hidden = relu(W1[h] x + b1[h])               (`hidden` values)
 *   psi    = W2[h] hidden + b2[h]                (2 head_dim values)
 *   phi(x) = [1 + elu(psi[0:d]), psi[d:2d]^2]    (D' = 2 head_dim, phi >= 0)
 *
 * The MLP's shape is a reading of the pages (Linear-ReLU-Linear with biases;
 * the degree-1 part made non-negative as 1 + elu, as §3.1 requires of phi).
 * bf16 calls: W1, W2 in bf16, products accumulated in fp32, the hidden layer
 * and phi rounded to bf16 (a bf16 model's activation precision); the linear
 * state is still accumulated in fp32.  fp32 calls: everything in fp32.
 * All pointers are device pointers, 16-byte aligned, owned by the caller.
 */
typedef struct rehyat_mlp_weights {
    const void* w1;   /* [H][hidden][head_dim], dtype of the call */
    const float* b1;  /* [H][hidden] fp32 */
    const void* w2;   /* [H][2 head_dim][hidden], dtype of the call */
    const float* b2;  /* [H][2 head_dim] fp32 */
    int hidden;       /* 32, 64, 128 or 256 (the same for the query and key maps) */
} rehyat_mlp_weights;

/* phi of every row: x [B][H][rows][head_dim] -> phi [B][H][rows][2 head_dim], both
 * in dtype (REHYAT_BF16 or REHYAT_F32); phi must not overlap x.  The map the
 * forward entry points below apply to q (with phi_q) and k (with phi_k). */
rehyat_status rehyat_feature_mlp(const void* x, void* phi, int dtype, int B, int H, int rows, int head_dim,
                                 const rehyat_mlp_weights* w, void* stream);

/* Forward with the learned maps: the contract of rehyat_attn_fwd (causal != 0)
 * or rehyat_attn_fwd_bidir (causal == 0), in dtype, with phi(q) = phi_q(q) and
 * phi(k) = phi_k(k).  The stream's workspace arena also holds phi(q) and phi(k)
 * (B H N 2 head_dim elements each). */
rehyat_status rehyat_attn_fwd_mlp(const void* q, const void* k, const void* v, void* out, int dtype,
                                  int B, int H, int frames, int tokens_per_frame, int head_dim,
                                  int chunk_frames, int overlap_frames, int causal,
                                  const rehyat_mlp_weights* phi_q, const rehyat_mlp_weights* phi_k,
                                  void* stream);
/* Per-query partials of the above (see rehyat_attn_fwd_partials). */
rehyat_status rehyat_attn_fwd_mlp_partials(const void* q, const void* k, const void* v, int dtype,
                                           float* m, float* nt, float* o_s, float* o_l, float* n_l,
                                           int B, int H, int frames, int tokens_per_frame, int head_dim,
                                           int chunk_frames, int overlap_frames, int causal,
                                           const rehyat_mlp_weights* phi_q,
                                           const rehyat_mlp_weights* phi_k, void* stream);
/* One streaming step with the learned maps, on a state initialised with
 * REHYAT_PHI_MLP2 (the state then also carries phi(k) of the overlap frames).
 * The same weights must be passed on every step of a stream. */
rehyat_status rehyat_attn_step_mlp(rehyat_step_state* st, const void* q, const void* k, const void* v,
                                   void* out, int frames, const rehyat_mlp_weights* phi_q,
                                   const rehyat_mlp_weights* phi_k, void* stream);

/*
 * Attention blocks (ReHyAt §3.1, first display equation: a DiT block is
 * T_l(x) = f_l(A_l(x) + x); §4.3 "Model Hyperparameters": 15, 20 or 25 of the
 * 30 blocks of Wan2.1 1.3B are converted to the hybrid attention).  The
 * attention part with its projections, on x [B][N][C] token-major bf16,
 * C = heads * head_dim, N = frames * tokens_per_frame:
 *   q = x Wq^T + bq,  k = (x Wk^T + bk) / sqrt(head_dim),  v = x Wv^T + bv,
 *   split into heads ([B][heads][N][head_dim], the attention layout);
 *   A(x) = concat_heads(attn(q, k, v)) Wo^T + bo;   output x + A(x).
 * attn is rehyat_attn_fwd with (chunk_frames, overlap_frames, feature_map) when
 * the block is hybrid, and full bidirectional softmax attention (one chunk
 * over the clip, no linear branch: the block before conversion) when not.
 * f_l (the rest of the DiT block) is not part of this; q/k normalisation and
 * rotary position embedding, which the pages do not describe, are not applied.
 * The projections run on bf16 MFMA with fp32 accumulation; q, k, v and the
 * attention output are bf16.  heads * head_dim must be a multiple of 128 and
 * B*N*C*2 bytes below 2^31.  Workspace (q, k, v, the attention output, the
 * attention's own workspace; two activation buffers for a stack) comes from
 * the stream's arena.  feature_map: NONE, ELU1 or POLY2.
 */
typedef struct rehyat_block_weights {
    const void* w_qkv;   /* [3C][C] bf16, out x in: rows 0..C-1 query, C..2C-1 key, 2C..3C-1 value */
    const float* b_qkv;  /* [3C] fp32 */
    const void* w_o;     /* [C][C] bf16, out x in */
    const float* b_o;    /* [C] fp32 */
} rehyat_block_weights;

/* One block: out = x + A(x) (hybrid != 0: ReHyAt attention, 0: full softmax).
 * out must not overlap x. */
rehyat_status rehyat_block_fwd(const void* x, void* out, const rehyat_block_weights* w, int B, int frames,
                               int tokens_per_frame, int heads, int head_dim, int hybrid, int chunk_frames,
                               int overlap_frames, int feature_map, void* stream);

/* A stack of n_blocks blocks, x_{l+1} = x_l + A_l(x_l) with weights w[l] and
 * hybrid[l] selecting each block's attention (host arrays of n_blocks
 * entries); out = x_{n_blocks}. */
rehyat_status rehyat_stack_fwd(const void* x, void* out, const rehyat_block_weights* w, const int* hybrid,
                               int n_blocks, int B, int frames, int tokens_per_frame, int heads, int head_dim,
                               int chunk_frames, int overlap_frames, int feature_map, void* stream);

/*
 * Training direction (ReHyAt §3.4: attention distillation and fine-tuning
 * backpropagate through the hybrid attention).  causal != 0 selects the
 * recurrent partition (rehyat_attn_fwd), causal == 0 the bidirectional one
 * (rehyat_attn_fwd_bidir); the backward must use the forward's choice.
 *
 * rehyat_attn_fwd_lse: the forward (dtype REHYAT_BF16 or REHYAT_F32) that also
 *   writes lse [B][H][N] fp32 = ln(n^S + n^L), the joint normaliser of each query,
 *   and, if out_f32 is not NULL (bf16 calls), the output before its rounding to
 *   bf16, fp32 [B][H][N][head_dim].
 * rehyat_attn_bwd uses out_f32 (may be NULL) rather than the bf16 out for the
 *   row sums D = dout . out.  The linear sums of the bidirectional form cancel
 *   in the gradient, which magnifies the bf16 rounding of out: there, dq drifts
 *   to ~1e-2 relative error from the rounded out alone at the Wan shape (the
 *   recurrent form: ~2e-4).
 * rehyat_attn_bwd: gradients of sum(dout * out) with respect to q, k and v, given
 *   the forward's inputs, out and lse, and dout (same shape and dtype as out).
 *   dq, dk, dv: caller-owned outputs in dtype, [B][H][N][head_dim], overlapping
 *   no input and no other gradient.  feature_map NONE, ELU1 or POLY2 (the learned
 *   map is not differentiated here).  The gradients of the linear branch flow
 *   through the same cached sums as the forward: the forward states S_t, z_t,
 *   and their reverse-order counterpart, sums over the chunks whose linear set
 *   holds a key's block (later chunks; bidirectional: later and earlier ones)
 *   of e^{-lse} phi(q) dout^T.  Workspace comes from the stream's arena.
 *   Deterministic: no atomics, fixed summation order.
 */
rehyat_status rehyat_attn_fwd_lse(const void* q, const void* k, const void* v, void* out, float* lse,
                                  float* out_f32, int dtype, int B, int H, int frames, int tokens_per_frame,
                                  int head_dim, int chunk_frames, int overlap_frames, int feature_map,
                                  int causal, void* stream);
rehyat_status rehyat_attn_bwd(const void* q, const void* k, const void* v, const void* out, const float* out_f32,
                              const float* lse, const void* dout, void* dq, void* dk, void* dv, int dtype,
                              int B, int H, int frames, int tokens_per_frame, int head_dim, int chunk_frames,
                              int overlap_frames, int feature_map, int causal, void* stream);

/*
 * Profiling aid.  While set on the calling thread, every whole-clip forward
 * call records four hipEvent_t handles on its stream: events[0] before the
 * block-state kernel, events[1] before the scan kernel, events[2] before the
 * local-softmax kernel and events[3] after it (events[0..2] coincide when the
 * call has no linear branch).  Pass (NULL, 0) to stop.  The events are owned by
 * the caller and must stay valid until the calls that record them complete.
 * n_events must be 0 or 4.
 */
rehyat_status rehyat_set_profile_events(void* const* events, int n_events);

/*
 * Waits for the work queued on `stream` (on the current device) and frees the
 * workspace arena of that stream and its side stream.  The next call on the
 * stream allocates new ones.  Must not run concurrently with a call on the same
 * stream.
 */
rehyat_status rehyat_workspace_release(void* stream);

/*
 * Test hook (fault injection).  Every HIP runtime call and kernel launch that
 * an entry point makes counts as one HIP step, numbered from 0 per call on the
 * calling thread.  rehyat_debug_inject_hip_error(n) arms the hook: the next
 * call that reaches step n returns REHYAT_EHIP at that step without making
 * the HIP call (so nothing after it is queued), and the hook disarms.  n < 0
 * disarms it.  rehyat_debug_hip_steps() returns the number of HIP steps the
 * last call on this thread made (or attempted).
 */
void rehyat_debug_inject_hip_error(int step);
int rehyat_debug_hip_steps(void);

/* Static description of a status code. */
const char* rehyat_status_string(int status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* rehyat_last_error(void);

/* Library version string. */
const char* rehyat_version(void);

#ifdef __cplusplus
}
#endif

#endif /* REHYAT_H */
