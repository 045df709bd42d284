/*
 * la.h -- C ABI of the MI355X (gfx950) ReLU linear-attention token mixer.
 *
 * The operation is the one defined on the SANA-Video analysis page
 * (arXiv 2509.24695, section 3.4 "Detailed, Sentence-Based Technical
 * Breakdown"):
 *
 *   "ReLU Linear Attention Mechanism" (unnumbered equation) with RoPE as in
 *   "Integration of 3D Rotary Position Embeddings", Eq. 2:
 *
 *     S = sum_j RoPE(relu(K_j))^T V_j          (d x d per (batch, head))
 *     z = sum_j relu(K_j)                       (d, NOT rotated)
 *     O_i = RoPE(relu(Q_i)) S / (relu(Q_i) . z + eps)
 *
 *   and "Block Linear Attention with Constant-Memory KV Cache" (Eq. 3, the
 *   running-sum update, Table 1, Algorithm 1): S and z are carried from block
 *   to block; block b is applied with the sums over blocks 0..b.  Eq. 3 taken
 *   token by token is the token-causal mode (la_token_causal).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Q, K, V, O are contiguous [B, H, n, d] arrays in device memory, element
 *    type `dtype` (LA_BF16 = bfloat16, LA_FP32 = float).  n is N for the
 *    bidirectional and token-causal calls and the block's length for
 *    la_block_causal_step.
 *  - S is a contiguous [B, H, d, d] float array, row index = key channel,
 *    column index = value channel.  z is a contiguous [B, H, d] float array.
 *    Both are always fp32 and always caller-owned device memory.
 *  - d must be 32, 64, 112 or 128 (112: SANA-Video-2B's head size, section
 *    3.4 "Macro-architecture specifications (Table 6)").  eps >= 0 is added
 *    to the denominator only.
 *    A row whose relu(Q_i) is all zero gets an all-zero output row.
 *  - (gt, gh, gw) is the latent grid.  Token n sits at
 *    t = n / (gh*gw), h = (n / gw) % gh, w = n % gw (0-based, t-major).
 *    gt = gh = gw = 0 switches RoPE off; otherwise all three must be >= 1 and
 *    gt*gh*gw >= N.  The d/2 interleaved channel pairs (2p, 2p+1) are split
 *    into t, h, w ranges of d/2 - 2*floor(d/6), floor(d/6), floor(d/6) pairs;
 *    pair k of an axis with P_a pairs turns by pos_a * 10000^(-k/P_a).
 *  - ws is a device workspace of at least la_workspace_bytes(B, H, N, d)
 *    bytes (la_workspace_bytes_grid() for a given grid): per-head counters,
 *    the per-workgroup partial states of the state pass and, in block mode,
 *    the block's sums.  Zero-fill it ONCE before its first use (e.g. right
 *    after allocating it).  The counters carry the epoch of the call that
 *    last used them (an increasing per-process number), so no call needs to
 *    reset them and a call that never completed leaves nothing a later call
 *    misreads (the epoch is a 32-bit count of calls in this process: such a
 *    leftover could be misread only by a call 2^32 calls later).  One workspace must not be used by two calls that may overlap
 *    in time (two streams): they would race on it.  Calls check ws_bytes
 *    against their own plan and return LA_E_WORKSPACE if it is too small.
 *  - All pointers must be 16-byte aligned.  O must not overlap Q, K, V, S or
 *    z, and ws must not overlap any other buffer of the call (LA_E_ALIAS).
 *  - stream is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues kernels: it never allocates, never synchronises, and returns as
 *    soon as the launches are queued.
 *  - Return value: LA_OK or a negative LA_E_* code.  Argument checks run
 *    before any launch; when one fails nothing is launched and no buffer is
 *    touched.  LA_E_HIP means a launch was rejected by the HIP runtime.
 *    Non-finite inputs are not checked: they propagate.
 */
#ifndef LA_H
#define LA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define LA_API __attribute__((visibility("default")))
#else
#define LA_API
#endif

enum { LA_FP32 = 0, LA_BF16 = 1 };

enum {
    LA_OK = 0,
    LA_E_NULLPTR = -1,     /* a required pointer is NULL */
    LA_E_SHAPE = -2,       /* bad B/H/N/grid/block arguments */
    LA_E_UNSUPPORTED = -3, /* d not in {32,64,112,128}, bad dtype, grid too large */
    LA_E_ALIGN = -4,       /* a pointer is not 16-byte aligned */
    LA_E_WORKSPACE = -5,   /* ws_bytes < la_workspace_bytes(...) */
    LA_E_HIP = -6,         /* the HIP runtime rejected a launch */
    LA_E_ALIAS = -7        /* O overlaps an input */
};

/* Workspace bytes that every call below needs for these sizes, N = tokens
 * of the whole sequence (largest partial count any of their plans chooses
 * in either dtype, with the tuning knobs as they are set now).  Calls with
 * RoPE on a grid whose table forces smaller chunks -- long sequences on
 * grid planes of a few positions -- can need more: la_workspace_bytes_grid
 * covers those.  Returns 0 for invalid sizes. */
LA_API size_t la_workspace_bytes(int B, int H, int N, int d);
LA_API size_t la_workspace_bytes_grid(int B, int H, int N, int d, int gt, int gh, int gw);

/* State pass (the two sums of the linear-attention equation, Eq. 2 form):
 *   S[b,h] = sum_{n<N} RoPE(relu(K[b,h,n]))^T V[b,h,n],  z[b,h] = sum_n relu(K[b,h,n]).
 * Reads K and V; writes S and z.  Q and O are not used and may be NULL;
 * block_tokens is ignored.  N = 0 gives S = 0, z = 0 (K, V may then be NULL).  The sum is split over many workgroups and
 * combined in a fixed order, so repeated calls give bitwise equal results. */
LA_API int la_state_reduce(const void* Q, const void* K, const void* V, void* O,
                    float* S, float* z, void* ws, size_t ws_bytes,
                    int B, int H, int N, int d, int gt, int gh, int gw,
                    int block_tokens, float eps, int dtype, void* stream);

/* The state pass as la_state_reduce, for callers that cannot allocate device
 * memory -- code under stream capture, tight serving loops, harnesses that
 * forbid allocation -- and so have no workspace to pass: its counters and
 * partial states live in a static array of the library (one per GPU, held
 * until the process ends) of LA_NOALLOC_SCRATCH_BYTES bytes.  Same arguments,
 * kernels and results (bitwise) as la_state_reduce without ws / ws_bytes.
 * Sizes whose plan needs more scratch than that return LA_E_WORKSPACE before
 * anything is launched (la_last_hip_error() then says how much they need).
 * The call allocates nothing and calls no allocating routine.  The first call
 * on a device looks up the array's address there and clears its counters on
 * `stream` (inside a stream capture that clear becomes part of the graph,
 * which is harmless: the counters are zero between completed calls).  Every
 * call on one GPU shares that GPU's array: two calls that may overlap in
 * time (two streams, two threads) race on it and must not be made; calls in
 * order on one stream are safe. */
#define LA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
LA_API int la_state_reduce_noalloc(const void* Q, const void* K, const void* V, void* O,
                            float* S, float* z,
                            int B, int H, int N, int d, int gt, int gh, int gw,
                            int block_tokens, float eps, int dtype, void* stream);

/* Apply pass (numerator / denominator of Eq. 2):
 *   O[b,h,n] = RoPE(relu(Q[b,h,n])) S[b,h] / (relu(Q[b,h,n]) . z[b,h] + eps).
 * Reads Q, S, z; writes O (bf16 outputs are rounded to nearest even).
 * K and V are not used and may be NULL; block_tokens is ignored.  ws is not
 * used by this call and may be NULL (ws_bytes is then ignored).  N = 0 is a
 * no-op that returns LA_OK after the argument checks on sizes. */
LA_API int la_apply(const void* Q, const void* K, const void* V, void* O,
             const float* S, const float* z, void* ws, size_t ws_bytes,
             int B, int H, int N, int d, int gt, int gh, int gw,
             int block_tokens, float eps, int dtype, void* stream);

/* Linear cross-attention in one call (the SANA-Video analysis page, "How
 * SANA-Video Positions Itself" and the Linear DiT block of section 3.4: the
 * cross-attention is the same ReLU linear attention as Eq. 2; text tokens
 * carry no grid position, so no RoPE):
 *   O[b,h,i] = relu(Q[b,h,i]) S[b,h] / (relu(Q[b,h,i]) . z[b,h] + eps),
 *   S[b,h] = sum_j relu(K[b,h,j])^T V[b,h,j],   z[b,h] = sum_j relu(K[b,h,j]),
 * over the N_kv keys/values.  Q, O: [B, H, N_q, d]; K, V: [B, H, N_kv, d]
 * (K and V may be NULL when N_kv = 0: O is then all zeros).  bf16 at d = 64
 * with N_kv <= 512 runs as one launch, each apply workgroup forming its
 * heads' S and z from K and V; every other case runs the state pass into
 * the workspace's S and z, then the apply pass (la_state_reduce and
 * la_apply in one call).  ws: at least la_cross_workspace_bytes(B, H, N_kv,
 * d) bytes, zero-filled once like any workspace, used only by the two-launch
 * path; it must not overlap Q, K, V or O, nor O overlap Q, K or V
 * (LA_E_ALIAS).  N_q = 0 returns LA_OK with nothing written.  Each output
 * has one fixed order of summation, so repeated calls give bitwise equal
 * results. */
LA_API int la_cross_attention(const void* Q, const void* K, const void* V, void* O,
                       void* ws, size_t ws_bytes, int B, int H, int N_q, int N_kv, int d,
                       float eps, int dtype, void* stream);

/* Workspace bytes for la_cross_attention over N_kv keys/values (0 for
 * invalid sizes). */
LA_API size_t la_cross_workspace_bytes(int B, int H, int N_kv, int d);

/* One block of block-causal mode (Eq. 3 taken a block at a time, Algorithm 1).
 * The sequence has N tokens in blocks of L = block_tokens; block b =
 * block_idx covers global tokens [b*L, min((b+1)*L, N)) and Q, K, V, O hold
 * only that block: [B, H, L_b, d] with L_b = min(L, N - b*L).
 * On entry S_carry/z_carry hold the sums over blocks < b (zero-filled before
 * block 0: the empty cache).  The call forms S_b = S_carry + (block b's sum),
 * z_b likewise, applies them to block b's rows with RoPE at the global
 * positions, and writes O.  commit = 1 stores S_b, z_b back into
 * S_carry/z_carry (the cache update after the clean block); commit = 0 leaves
 * the carry untouched (a denoising step that only reads the cache). */
LA_API int la_block_causal_step(const void* Q, const void* K, const void* V, void* O,
                         float* S_carry, float* z_carry, void* ws, size_t ws_bytes,
                         int B, int H, int N, int d, int gt, int gh, int gw,
                         int block_tokens, float eps, int dtype,
                         int block_idx, int commit, void* stream);

/* Token-causal mode (Eq. 3 literally: section 3.3.1 of the same page,
 * "Derivation from causal linear attention"; RoPE as in Eq. 2): token i sees
 * tokens j <= i of the sequence,
 *   S_i = S_carry + sum_{j<=i} RoPE(relu(K_j))^T V_j,   z_i = z_carry + sum_{j<=i} relu(K_j),
 *   O_i = RoPE(relu(Q_i)) S_i / (relu(Q_i) . z_i + eps).
 * Q, K, V, O are [B, H, N, d]; token i sits at global position n_offset + i
 * (gt*gh*gw must hold n_offset + N tokens), so a long sequence can be fed in
 * segments.  S_carry/z_carry are both NULL (start from the empty state; the
 * final state is not returned) or both non-NULL: the state before token 0 on
 * entry, the state after token N-1 on return.  Every d and dtype of the
 * other calls (bf16 on matrix cores, fp32 in plain fp32 arithmetic).
 * N = 0 returns LA_OK and leaves the carry as
 * it is.  ws: at least la_workspace_bytes(B, H, N, d) bytes (this call
 * neither needs nor disturbs the zero counters); it must not overlap O or
 * the carry.  Every piece of
 * the computation has a fixed order, so repeated calls give bitwise equal
 * results. */
LA_API int la_token_causal(const void* Q, const void* K, const void* V, void* O,
                    float* S_carry, float* z_carry, void* ws, size_t ws_bytes,
                    int B, int H, int N, int d, int gt, int gh, int gw, int n_offset,
                    float eps, int dtype, void* stream);

/* One block of the block-causal temporal convolution of the Mix-FFN, with
 * its shortcut (same page, section 3.4, "Spatial-Temporal Mix-FFN" and
 * "Block Causal Mix-FFN", Figure 4(b)).  Per spatial position p:
 *   Y[b,f,p] = X[b,f,p] + W[0] X[b,f-1,p] + W[1] X[b,f,p] + W[2] X[b,f+1,p] (+ bias)
 * for the block's frames f = 0..T-1, where X[b,-1,p] = cache[b,p] (the last
 * frame of the previous block: zero-fill the cache before the first block)
 * and X[b,T,p] = 0 (zero padding: no block sees a later one).  W[k] x is the
 * matrix-vector product with the D x D matrix W[k] (row = output channel).
 *  - X, Y: contiguous [B, T, P, D] bf16 (frame-major tokens, P spatial
 *    positions per frame, D channels).  W: contiguous [3, D, D] bf16,
 *    W[k][out][in].  bias: [D] float or NULL.  cache: [B, P, D] bf16.
 *    All device memory, caller-owned, 16-byte aligned.
 *  - commit = 1 writes X[b, T-1] into cache[b] after Y is formed (the cache
 *    update after the clean block); commit = 0 leaves the cache untouched.
 *  - Products run in bf16 with fp32 accumulation; Y is rounded to nearest
 *    even once, after the shortcut and bias are added.
 *  - dtype must be LA_BF16, D a multiple of 64 and at most 16384, and X
 *    under 2 GiB (otherwise LA_E_UNSUPPORTED: split a larger call by
 *    batch).  B*T*P = 0 returns LA_OK with nothing written.  Y must not
 *    overlap X, W, bias or cache, nor the cache X, W or bias (LA_E_ALIAS).
 *  - No workspace; the call only enqueues kernels on stream.  Every output
 *    element has one fixed order of summation, so repeated calls give
 *    bitwise equal results. */
LA_API int la_temporal_conv_step(const void* X, void* Y, const void* W, const float* bias, void* cache,
                                 int B, int T, int P, int D, int commit, int dtype, void* stream);

/* Measurement utility, not part of the method: a plain copy of `bytes`
 * bytes from src to dst (device memory, 16-byte aligned, bytes a multiple of
 * 16, no overlap; otherwise LA_E_ALIGN / LA_E_ALIAS), one 16-byte piece per
 * lane, with the same cache policies as the kernels' own streams
 * (non-temporal loads, streaming stores).  Its rate is the practical ceiling
 * of a read + write HBM stream that the kernels above are compared with.  bytes = 0 returns LA_OK; more than
 * 2^42 bytes returns LA_E_UNSUPPORTED. */
LA_API int la_stream_copy(const void* src, void* dst, size_t bytes, void* stream);

/* Measurement only, not part of the method: set a tuning knob of this
 * process's library instance, for A/B runs on one build.  Knobs (value < 0
 * restores the default choice, which is what every figure quoted for this
 * library uses):
 *   "state_wgs", "apply_wgs", "causal_wgs"  target workgroup counts (>= 1)
 *   "state_fused"      0 / 1: separate / in-kernel stage 2 of the state pass
 *   "apply_ilv"        0: one contiguous chunk per apply workgroup
 *   "apply_heads"      1..8: heads per apply slot (if they divide B*H and fit)
 *   "tc_state_threads" 512 / 1024: token-causal partial-state workgroups
 *   "tconv_gm", "tconv_gn"  temporal-convolution tile-order group (1..64)
 *   "apply_spread"     0 / 1: a slot's apply workgroups on as few XCDs as possible / on all 8
 *   "cross_fused"      0: la_cross_attention always takes the two-launch path
 * Returns LA_OK, LA_E_NULLPTR, LA_E_UNSUPPORTED (unknown name) or
 * LA_E_SHAPE (value out of range).  Not thread-safe: set knobs while no
 * other thread calls the library.  Results are correct under every value. */
LA_API int la_set_tuning(const char* name, int value);

/* Static text for a status code (never NULL). */
LA_API const char* la_strerror(int status);

/* After LA_E_HIP: the failing HIP call, error name, code and description, as
 * seen by the calling thread ("" if no HIP call has failed on this thread).
 * The text stays valid until the thread's next failing call. */
LA_API const char* la_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LA_H */
