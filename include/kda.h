/*
 * kda.h -- C ABI of the KDA (Kimi Delta Attention) token mixer for AMD MI355X (gfx950).
 *
 * The operation.  KDA is a gated delta rule with one retention factor per key channel.  For each
 * sequence and head the state S is a dk x dv matrix ("Kimi K3's hybrid block, from first
 * principles", section "From linear attention to the delta rule": the state is dk x dv and the
 * same size at every token; K3 uses dk = dv = 128 and 96 heads, paragraph "What the state
 * costs").  Token by token, with alpha_t = exp(g_t) in (0,1]^dk:
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,     o_t = S_t^T q_t
 *
 * i.e. fade every key channel by its own factor, then remove what the memory returns for k_t and
 * write v_t (a gradient step of size beta_t on 1/2 |S^T k_t - v_t|^2), then read the updated
 * state with q_t ("Kimi K3, explained", section "Kimi Delta Attention: making the radical option
 * work": fade, remove, write; q reads the updated S(t); "What's new in Kimi K3", section "KDA in
 * one page": the forget gate sits in front of the erase).  No query scaling is applied.
 *
 * Number formats.  q, k, v, g, beta and o are all bfloat16 (KDA_BF16) or all float32 (KDA_F32);
 * states (h0, hT, S) are always float32; arithmetic is float32 (bf16 matrix-core products with
 * float32 accumulation on the bf16 path).
 *
 * Layouts.  Row-major, contiguous, token-major ("packed"):
 *     q, k, g : [Ttot, H, dk]     v, o : [Ttot, H, dv]     beta : [Ttot, H]
 *     h0, hT, S : [N, H, dk, dv]  (float32; S row r = key channel r)
 * Ttot = B * T for B equal-length sequences (cu_seqlens == NULL; sequence b owns tokens
 * b*T .. b*T+T-1) or the packed total for a variable-length batch (cu_seqlens != NULL, B == 1).
 *
 * Preconditions (documented, not checked unless the environment variable KDA_VALIDATE=1 is set
 * when the call is made): g in [-5, 0] -- the pages' bounded log-decay ("Kimi K3", section
 * "Forgetting different features at different rates": retention never falls below e^-5, which
 * keeps the tile rescaling factors of the chunked algorithm finite); cu_seqlens non-decreasing
 * with cu[0] = 0 and cu[N] = Ttot.  q and k are expected L2-normalised upstream but the result is
 * defined for any values.  NaN/Inf inputs propagate; they are not checked.
 *
 * Ownership and streams.  The caller owns every buffer (device memory, e.g. allocated by PyTorch)
 * and passes a HIP stream (hipStream_t as void*, NULL = the null stream).  The library allocates
 * nothing, keeps no state between calls and is thread-safe, with one exception:
 * kda_chunk_fwd_split_noalloc keeps its workspace in a static device array per GPU, which calls
 * that overlap on one GPU share.  Calls are asynchronous: the return
 * status reports argument errors and launch failures; execution faults surface at the caller's
 * next synchronisation of the stream.
 *
 * Graph capture.  Outside the validation mode (KDA_VALIDATE, which copies to the host and
 * synchronises), a compute entry point only enqueues kernels on the given stream: no allocation,
 * no synchronisation, no memset.  Calls may therefore be captured into a HIP graph and replayed
 * (the kernels read their inputs at replay time).  kda_chunk_fwd_split_noalloc looks up its
 * static array on its first call on a device: make that first call outside a capture.
 *
 * Supported sizes.  dk and dv: multiples of 16 from 16 to 128 (any combination).  The fast
 * matrix-core path is used for dtype KDA_BF16 with dk = dv = 128; every other supported
 * combination runs the general float32 tile path.  H >= 1 with H * max(dk, dv) <= 2^20 (one
 * token's row of a tensor; larger rows return KDA_ERR_SHAPE, since the streaming kernels address
 * a few dozen consecutive rows with 32-bit byte offsets); B, T, N >= 0 (empty input is a no-op
 * that still copies h0 to hT).
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dtype of q, k, v, g, beta and o */
typedef enum { KDA_BF16 = 0, KDA_F32 = 1 } kda_dtype;

/* status codes (0 = success) */
enum {
    KDA_OK = 0,
    KDA_ERR_NULL = -1,        /* a required pointer is NULL */
    KDA_ERR_SHAPE = -2,       /* negative or inconsistent sizes, or H * max(dk, dv) > 2^20 */
    KDA_ERR_DTYPE = -3,       /* dtype not KDA_BF16 / KDA_F32 */
    KDA_ERR_UNSUPPORTED = -4, /* dk or dv not a multiple of 16 in [16, 128] */
    KDA_ERR_SEQLENS = -5,     /* cu_seqlens with B != 1, or (KDA_VALIDATE) bad contents */
    KDA_ERR_RANGE = -6,       /* (KDA_VALIDATE) g outside [-5, 0]; or eps < 0 */
    KDA_ERR_HIP = -7,         /* a HIP runtime call or kernel launch failed */
    KDA_ERR_STRIDE = -8,      /* snapshot stride not a positive multiple of 16, or (KDA_VALIDATE)
                                 snap_offsets inconsistent with the sequence lengths */
    KDA_ERR_ALIGN = -9,       /* a buffer of the output stage is not 16-byte aligned */
    KDA_ERR_WORKSPACE = -10,  /* workspace NULL, smaller than the size query returns, or not
                                 256-byte aligned */
    KDA_ERR_SCRATCH = -11     /* the call needs more workspace than the library's static device
                                 array holds (kda_chunk_fwd_split_noalloc: 32 MiB per device) */
};

/*
 * kda_chunk_fwd -- prefill: run the recurrence over whole sequences and return every output and
 * the final state.  Computed chunkwise, in parallel inside 16-token tiles and recurrently across
 * tiles ("Kimi K3's hybrid block, from first principles", section "From linear attention to the
 * delta rule": the tokens of a chunk are processed together and a state is passed from chunk to
 * chunk; with the -5 floor the summed log-decay of a 16-token tile lies in (-80, 0)).  The
 * chunked result equals the token loop up to floating-point rounding ("Kimi K3", section
 * "Forgetting different features at different rates").  Tiles restart at every sequence start; a sequence's last tile may be
 * partial.
 *
 *   q, k, g   [Ttot, H, dk]  dtype    device      inputs (g = log alpha, natural log)
 *   v         [Ttot, H, dv]  dtype    device
 *   beta      [Ttot, H]      dtype    device      write strength per token and head
 *   h0        [N, H, dk, dv] float32  device      initial states; NULL = zeros
 *   cu_seqlens [N+1]         int32    device      NULL = B equal sequences of length T
 *   num_seqs  N (used only with cu_seqlens; else N = B)
 *   o         [Ttot, H, dv]  dtype    device      output (written)
 *   hT        [N, H, dk, dv] float32  device      final states (written); NULL = not written.
 *                                                 hT may alias h0 (in-place state update).
 *   B, T      with cu_seqlens: B must be 1 and T = Ttot; else Ttot = B * T
 *   H, dk, dv heads and head dimensions
 *   dtype     kda_dtype
 *   stream    hipStream_t as void*
 * Returns KDA_OK or a negative status; nothing is written on an argument error.
 */
int kda_chunk_fwd(const void* q, const void* k, const void* v, const void* g, const void* beta,
                  const float* h0, const int32_t* cu_seqlens, int num_seqs,
                  void* o, float* hT,
                  int B, int T, int H, int dk, int dv, int dtype, void* stream);

/*
 * kda_chunk_fwd_gated -- kda_chunk_fwd followed by the output stage of kda_output_gate on its
 * outputs: y[t,h,:] = o[t,h,:] / sqrt(mean_c o[t,h,c]^2 + eps) * weight * sigmoid(gate[t,h,:])
 * ("Kimi K3's hybrid block, from first principles", section "From linear attention to the delta
 * rule": each head's output row is normalised by its root mean square and scaled by a sigmoid
 * gate of the token before the output projection).  For bf16 with dk = dv = 128 and at least
 * 256 (sequence, head) pairs (kda_chunk_fwd_gated_fuses) the stage runs inside the prefill
 * kernel, on each tile's outputs while they are still on chip: o is then written only if asked
 * for, and never read back.  Otherwise the prefill writes o (into y when o is NULL) and the
 * output stage runs after it.  The norm is taken over o as rounded to dtype, as kda_output_gate
 * would read it.
 *
 *   arguments as kda_chunk_fwd, plus
 *   gate      [Ttot, H, dv]  dtype    device      the gate's pre-activation per output element
 *   weight    [dv]           float32  device      the norm's gain per value channel; NULL = ones
 *   eps       >= 0 (KDA_ERR_RANGE otherwise)
 *   o         [Ttot, H, dv]  dtype    device      the mixer output (written); NULL = not wanted
 *   y         [Ttot, H, dv]  dtype    device      the gated output (written)
 * gate, y and o (when given) must be 16-byte aligned (KDA_ERR_ALIGN); y may alias o or gate.
 * Returns KDA_OK or a negative status; nothing is written on an argument error.
 */
int kda_chunk_fwd_gated(const void* q, const void* k, const void* v, const void* g,
                        const void* beta, const float* h0, const int32_t* cu_seqlens,
                        int num_seqs, const void* gate, const float* weight, float eps, void* o,
                        void* y, float* hT, int B, int T, int H, int dk, int dv, int dtype,
                        void* stream);

/*
 * kda_chunk_fwd_gated_fuses -- 1 when kda_chunk_fwd_gated runs the output stage inside the
 * prefill kernel for these arguments (varlen != 0: N = num_seqs, else N = B), else 0.
 */
int kda_chunk_fwd_gated_fuses(int num_seqs, int B, int H, int dk, int dv, int dtype, int varlen);

/*
 * kda_chunk_fwd_chunk64 -- kda_chunk_fwd computed with 64-token chunks made of four 16-token
 * sub-tiles: the state is carried once per chunk, and the chunk's 64x64 triangular system is
 * solved by blocks, the diagonal sub-tiles on their own and the coupling between sub-tiles as
 * separate off-diagonal products ("What's new in Kimi K3", section "KDA in one page": the
 * per-token cost is quoted at chunk size 64; "Kimi K3's hybrid block, from first principles",
 * section "From linear attention to the delta rule": the cumulative log-decay over 16 tokens
 * stays within (-80, 0), so every exponent is kept within one sub-tile or made non-positive).
 * bf16 with dk = dv = 128 runs on the matrix cores in two kernels: the state-independent part of
 * every (chunk, head) in parallel, written to the workspace, then the serial carry per (sequence,
 * head).  Other dtypes and head sizes run in float32 on the vector ALUs and need no workspace.
 * Same arguments, layouts, results (up to rounding) and errors as kda_chunk_fwd, plus
 *   workspace        device memory of at least kda_chunk_fwd_chunk64_workspace_bytes(...) bytes,
 *                    256-byte aligned, owned by the caller; its contents on entry do not matter
 *                    and are undefined on return; it may be NULL when that size is 0
 *   workspace_bytes  its size
 * KDA_ERR_WORKSPACE when the workspace is missing, too small or misaligned.
 */
int kda_chunk_fwd_chunk64(const void* q, const void* k, const void* v, const void* g,
                          const void* beta, const float* h0, const int32_t* cu_seqlens,
                          int num_seqs, void* o, float* hT,
                          int B, int T, int H, int dk, int dv, int dtype,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_chunk_fwd_chunk64_workspace_bytes -- bytes of workspace kda_chunk_fwd_chunk64 needs for
 * these arguments (only whether cu_seqlens is NULL matters; its contents are not read): 0 for the
 * float32 path; for the matrix-core path, 80.5 KiB per (64-token chunk, head) plus the chunk
 * offsets of a variable-length batch.  0 as well for arguments kda_chunk_fwd_chunk64 rejects.
 */
size_t kda_chunk_fwd_chunk64_workspace_bytes(const int32_t* cu_seqlens, int num_seqs, int B,
                                             int T, int H, int dk, int dv, int dtype);

/*
 * kda_chunk_fwd_split -- kda_chunk_fwd with each sequence also cut into token ranges that run at
 * the same time, for batches too small to fill the chip (one GPU's share of the heads at batch 1,
 * for instance).  The recurrence ("Kimi K3's hybrid block, from first
 * principles", section "From linear attention to the delta rule") is affine in the state, so any
 * run of tokens maps its entering state S to M S + B, and a segment that starts from an unknown
 * state S_in has S_t = M_t S_in + B_t.  Segment 0 runs from h0; every later
 * segment runs twice in the same launch, from a zero state with its values (B_t, outputs
 * B_t^T q_t) and from the identity with v = 0 (M_t, outputs M_t^T q_t).  A composition step then
 * chains S_in(s + 1) = M_s S_in(s) + B_s, writes hT, and adds S_in(s)^T (M_t^T q_t) to the outputs
 * of segment s.  About twice the state work of the later segments buys a serial chain of T / P
 * tokens instead of T.
 *
 * Arguments as kda_chunk_fwd, plus
 *   max_seqlen       with cu_seqlens: the length the segment plan assumes for the longest
 *                    sequence (the caller's bound; >= 0, 0 = no split).  Every sequence is cut
 *                    into segments of the planned length, the last running to its end, so a
 *                    bound below a real length costs speed, not correctness.  Ignored without
 *                    cu_seqlens (the plan uses T)
 *   segments         the number of token ranges P requested (at most 16); 0 lets the library
 *                    choose (kda_chunk_fwd_split_segments).  Segments are a multiple of 64
 *                    tokens, so fewer may be used than requested
 *   workspace        device memory of at least kda_chunk_fwd_split_workspace_bytes(...) bytes,
 *                    256-byte aligned, owned by the caller; contents on entry do not matter and
 *                    are undefined on return; may be NULL when that size is 0
 *   workspace_bytes  its size
 * The split applies to KDA_BF16 with dk = dv = 128 and N * H <= 65535; otherwise, or when one
 * segment results, the call is kda_chunk_fwd and needs no workspace.  Results equal
 * kda_chunk_fwd's up to rounding (the outputs of later segments are rounded to bf16 twice).
 * Returns KDA_OK, KDA_ERR_SHAPE for segments < 0 or max_seqlen < 0 with cu_seqlens,
 * KDA_ERR_WORKSPACE, or kda_chunk_fwd's errors.
 */
int kda_chunk_fwd_split(const void* q, const void* k, const void* v, const void* g,
                        const void* beta, const float* h0, const int32_t* cu_seqlens,
                        int num_seqs, int max_seqlen, void* o, float* hT,
                        int B, int T, int H, int dk, int dv, int dtype, int segments,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_chunk_fwd_split_segments -- the number of segments kda_chunk_fwd_split plans for these
 * arguments and request (1: no split; only whether cu_seqlens is NULL matters, not its contents).
 * With segments = 0 it is the largest P whose 2 (2 P - 1) N H matrix-core workgroups hold one of
 * the 256 compute units each, with at least 256 tokens per segment of the planned length (T, or
 * max_seqlen with cu_seqlens), and 1 once 2 N H >= 128.
 */
int kda_chunk_fwd_split_segments(const int32_t* cu_seqlens, int num_seqs, int max_seqlen, int B,
                                 int T, int H, int dk, int dv, int dtype, int segments);

/*
 * kda_chunk_fwd_split_workspace_bytes -- bytes of workspace kda_chunk_fwd_split needs: 0 without
 * a split; else Ttot H 256 bytes (the M_t^T q_t outputs in bf16) rounded up to 256, plus
 * P * 2 * N * H * 64 KiB (the final states of both runs of every segment).
 */
size_t kda_chunk_fwd_split_workspace_bytes(const int32_t* cu_seqlens, int num_seqs,
                                           int max_seqlen, int B, int T, int H, int dk, int dv,
                                           int dtype, int segments);

/*
 * kda_chunk_fwd_split_noalloc -- kda_chunk_fwd_split for callers that cannot allocate device
 * memory: code under HIP stream capture, tight serving loops, harnesses that forbid hipMalloc.
 * The workspace is a static device array of the library, 32 MiB per device (KDA_ERR_SCRATCH for
 * a call whose kda_chunk_fwd_split_workspace_bytes exceeds it, returned before anything runs);
 * the call itself allocates nothing.  The array's device address is looked up once per device,
 * on the first call made with that device current (the stream must belong to the current
 * device).  Every call on one GPU shares that GPU's array: calls that overlap on one GPU (other
 * streams, other threads) race and must be serialised by the caller.  Its contents between calls
 * do not matter.
 *
 * Arguments, results and the other errors as kda_chunk_fwd_split, without workspace and
 * workspace_bytes.
 */
int kda_chunk_fwd_split_noalloc(const void* q, const void* k, const void* v, const void* g,
                                const void* beta, const float* h0, const int32_t* cu_seqlens,
                                int num_seqs, int max_seqlen, void* o, float* hT,
                                int B, int T, int H, int dk, int dv, int dtype, int segments,
                                void* stream);

/*
 * kda_chunk_fwd_snapshots -- kda_chunk_fwd that also saves the state at every multiple of
 * snap_stride tokens of each sequence, for prefix caching.  A KDA layer keeps one state that
 * summarises the whole prefix, so a cached prefix can be resumed only from a state saved at
 * exactly its boundary ("Kimi K3's hybrid block, from first principles", section "Gated MLA
 * without positions", paragraph "The cache, in bytes"); a float32 snapshot costs 64 KiB per head,
 * so strides below 64 tokens hold more bytes than the per-token cache they replace ("What's new in
 * Kimi K3", section "What it costs to serve").  Passing a snapshot as h0 of a later call resumes
 * the sequence after that prefix.
 *
 * Arguments as kda_chunk_fwd, plus
 *   snaps        [Nsnap, H, dk, dv] float32 device   written: snapshot j (j = 1 .. len_n / snap_stride,
 *                                                    rounded down) of sequence n is the state after
 *                                                    its first j * snap_stride tokens, at index
 *                                                    snap_offsets[n] + j - 1
 *   snap_offsets [N+1] int32 device   snap_offsets[0] = 0 and snap_offsets[n+1] - snap_offsets[n] =
 *                                     len_n / snap_stride (rounded down); required with
 *                                     cu_seqlens; NULL without it (then index n * (T / snap_stride)
 *                                     + j - 1)
 *   snap_stride  a positive multiple of 16 (the tile size), else KDA_ERR_STRIDE
 * snaps = NULL is KDA_ERR_NULL when some sequence has snap_stride tokens or more (known from T
 * without cu_seqlens; checked from the offsets with KDA_VALIDATE=1), and otherwise writes nothing,
 * so an empty snapshot buffer may be passed as NULL.  With KDA_VALIDATE=1 the offsets are checked
 * against cu_seqlens (KDA_ERR_STRIDE).  Returns KDA_OK or a negative status.
 */
int kda_chunk_fwd_snapshots(const void* q, const void* k, const void* v, const void* g,
                            const void* beta, const float* h0, const int32_t* cu_seqlens,
                            int num_seqs, void* o, float* hT, float* snaps,
                            const int32_t* snap_offsets, int snap_stride,
                            int B, int T, int H, int dk, int dv, int dtype, void* stream);

/*
 * kda_decode_step -- one token for each of N sequences, updating their states in place and
 * returning the outputs: S <- (I - beta k k^T) Diag(exp g) S + beta k v^T, o = S^T q ("Kimi K3,
 * explained", section "Kimi Delta Attention: making the radical option work": one KDA token
 * step; k and v update S(t-1), q reads the updated S(t); "Kimi K3's hybrid block, from first
 * principles", paragraph "What the state costs": the same work at every token).
 *
 *   q, k, g   [N, H, dk]      dtype    device
 *   v         [N, H, dv]      dtype    device
 *   beta      [N, H]          dtype    device
 *   S         [N, H, dk, dv]  float32  device      read, then overwritten with the new state
 *   o         [N, H, dv]      dtype    device      output (written)
 * Returns KDA_OK or a negative status.
 */
int kda_decode_step(const void* q, const void* k, const void* v, const void* g, const void* beta,
                    float* S, void* o, int N, int H, int dk, int dv, int dtype, void* stream);

/*
 * kda_output_gate -- the output stage after the mixer: every (token, head) row of dv outputs is
 * RMS-normalised and multiplied by a sigmoid gate of the token ("Kimi K3's hybrid block, from first
 * principles", section "From linear attention to the delta rule": each head's output row is
 * normalised by its root mean square and scaled, ahead of the output projection, by a sigmoid gate
 * computed from the token at full rank):
 *
 *     y[t,h,:] = o[t,h,:] / sqrt(mean_c o[t,h,c]^2 + eps) * weight * sigmoid(gate[t,h,:])
 *
 *   o, gate, y [Ttot, H, dv]  dtype    device   16-byte aligned; y may alias o or gate
 *   weight     [dv]           float32  device   the norm's gain per value channel; NULL = ones
 *   eps        >= 0 (KDA_ERR_RANGE otherwise); an all-zero row with eps = 0 gives NaN
 *   Ttot, H, dv               tokens, heads, head size (dv a multiple of 16 in [16, 128])
 * Returns KDA_OK or a negative status.
 */
int kda_output_gate(const void* o, const void* gate, const float* weight, float eps, void* y,
                    int Ttot, int H, int dv, int dtype, void* stream);

/*
 * kda_decode_step_gated -- kda_decode_step followed by the output stage of kda_output_gate on its
 * outputs.  Writes both o and y.  For dk = dv = 128 (16-byte aligned S, 8-byte aligned v/o/gate/y
 * for bf16, 16-byte for float32) the stage runs inside the decode kernel, on the outputs while
 * they are still in registers; other sizes run the decode and then kda_output_gate.
 *
 *   arguments as kda_decode_step, plus gate [N, H, dv] (dtype), weight [dv] (float32 or NULL),
 *   eps >= 0 and y [N, H, dv] (dtype, written; may alias o or gate, which are then overwritten).
 * When the fused kernel does not apply, o, gate and y must be 16-byte aligned (KDA_ERR_ALIGN,
 * returned before anything runs).
 * Returns KDA_OK or a negative status.
 */
int kda_decode_step_gated(const void* q, const void* k, const void* v, const void* g,
                          const void* beta, float* S, const void* gate, const float* weight,
                          float eps, void* o, void* y, int N, int H, int dk, int dv, int dtype,
                          void* stream);

/*
 * kda_frontend -- the input stage before the mixer: turns the projected pre-activations of every
 * token into q, k, v, g and beta for kda_chunk_fwd / kda_decode_step ("Kimi K3's hybrid block,
 * from first principles", section "From linear attention to the delta rule": q and k get a
 * four-tap causal convolution, the Swish activation and unit-length normalisation, v the
 * convolution and Swish only; beta comes from a sigmoid over a projection of the token; the
 * log-decay has the floor g_min and one learned scale A_h per head).  Per token t, head h, channel c:
 *
 *     conv(x)[t,c] = sum_{i<4} w[c,i] x[t-3+i,c]     causal and depthwise; at a sequence start the
 *                                                   three earlier inputs come from conv_in (zeros
 *                                                   when conv_in is NULL)
 *     q = l2(swish(conv(x_q)))   k = l2(swish(conv(x_k)))   v = swish(conv(x_v))
 *     g = g_min * sigmoid(A[h] * (x_z + z_bias[c]))           beta = sigmoid(x_b)
 *     swish(y) = y * sigmoid(y);   l2(y) = y / sqrt(sum_c y_c^2 + eps) over the head's dk values
 *
 * The printed formula of the bounded gate is lost on the pages; this is the reading that matches
 * their statement (every retention factor between e^g_min and 1, one scale per head).
 *
 *   x_q, x_k, x_z [Ttot, H, dk], x_v [Ttot, H, dv], x_b [Ttot, H]   dtype    device  inputs
 *   w_q, w_k [H*dk, 4], w_v [H*dv, 4]      float32  device   taps; w[c,3] weighs the current token
 *   z_bias [H*dk], A [H]                   float32  device
 *   g_min (< 0), eps (>= 0)                                   else KDA_ERR_RANGE
 *   cu_seqlens, num_seqs, B, T             as kda_chunk_fwd (sequence boundaries)
 *   conv_in  [N, 3, H*(2dk+dv)]  dtype  device  the last three inputs of q | k | v before each
 *                                               sequence, oldest first; NULL = zeros
 *   conv_out [N, 3, H*(2dk+dv)]  dtype  device  written: the last three inputs of each sequence
 *                                               (rows of conv_in when shorter); NULL = not
 *                                               written; may alias conv_in (decode: one token per
 *                                               sequence with the state updated in place)
 *   q, k, g [Ttot, H, dk], v [Ttot, H, dv], beta [Ttot, H]   dtype  device  outputs
 * Every [*, H, d] buffer and the state rows must be 16-byte aligned (KDA_ERR_ALIGN).
 * Returns KDA_OK or a negative status.
 */
int kda_frontend(const void* x_q, const void* x_k, const void* x_v, const void* x_z,
                 const void* x_b, const float* w_q, const float* w_k, const float* w_v,
                 const float* z_bias, const float* A, float g_min, float eps,
                 const int32_t* cu_seqlens, int num_seqs, const void* conv_in, void* conv_out,
                 void* q, void* k, void* v, void* g, void* beta,
                 int B, int T, int H, int dk, int dv, int dtype, void* stream);

/*
 * kda_decode_step_layer -- the whole token mixer for one token per sequence in one launch: the
 * input stage of kda_frontend (decode mode, the convolution state updated in place), the decode
 * step of kda_decode_step (the recurrent state updated in place) and the output stage of
 * kda_output_gate ("Kimi K3's hybrid block, from first principles", section "From linear
 * attention to the delta rule": the short convolution, Swish and unit-length normalisation of q
 * and k, the bounded log-decay and the sigmoid beta before the recurrence, and the gated RMS
 * normalisation of each head's output row after it).  q, k, v, g and beta stay in float32 inside
 * the kernel, where kda_frontend followed by kda_decode_step_gated would store them in dtype.
 *
 *   x_q, x_k, x_z [N, H, dk], x_v [N, H, dv], x_b [N, H]   dtype    device  the token's
 *                                                         pre-activations
 *   w_q, w_k, w_v, z_bias, A, g_min, norm_eps            as kda_frontend (norm_eps: the L2 norms)
 *   conv_state [N, 3, H*(2dk+dv)]  dtype    device  the last three inputs of q | k | v before the
 *                                                  token, oldest first; read, then overwritten
 *                                                  with the three inputs that end at the token
 *   S          [N, H, dk, dv]      float32  device  read, then overwritten with the new state
 *   gate, weight, eps              as kda_decode_step_gated
 *   o          [N, H, dv]          dtype    device  written, or NULL (not written)
 *   y          [N, H, dv]          dtype    device  written; may alias o or gate
 * dk = dv = 128 only (KDA_ERR_UNSUPPORTED otherwise: other head sizes call kda_frontend, then
 * kda_decode_step_gated).  S 16-byte aligned; gate, o and y 8-byte aligned for bf16 and 16-byte
 * for float32 (KDA_ERR_ALIGN).  g_min < 0, norm_eps >= 0, eps >= 0 (KDA_ERR_RANGE).
 * Returns KDA_OK or a negative status.
 */
int kda_decode_step_layer(const void* x_q, const void* x_k, const void* x_v, const void* x_z,
                          const void* x_b, const float* w_q, const float* w_k, const float* w_v,
                          const float* z_bias, const float* A, float g_min, float norm_eps,
                          void* conv_state, float* S, const void* gate, const float* weight,
                          float eps, void* o, void* y, int N, int H, int dk, int dv, int dtype,
                          void* stream);

/* Text for a status code (static storage; never NULL). */
const char* kda_status_string(int status);

/* ABI version of this library (major * 10000 + minor * 100 + patch). */
int kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
