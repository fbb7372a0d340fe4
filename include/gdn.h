/*
 * gdn.h — C ABI of the MI355X (gfx950) gated delta-rule library (libgdn.so).
 *
 * The library computes the Gated DeltaNet linear-attention core
 *     S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,   o_t = scale * S_t^T q_t
 * with an fp32 d_k x d_v state per (sequence, head), and its per-key-channel (KDA-style)
 * variant S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T, in the two
 * forms the pages derive: a chunk-parallel prefill and a one-token recurrent decode, plus a
 * DeltaLog decode (dense base + append log) and the causal short convolution that precedes
 * the core.
 *
 * Sources (cited by page title and section):
 *   [LA-Infra]  "深度解析线性注意力机制演进与 AI Infra 实现" (todayforai.com)
 *   [Handbook]  "线性注意力与混合架构的推理" (AI-infra handbooks, anrans.github.io)
 *   [DeltaLog]  "DeltaLog：延迟物化递归状态以加速线性注意力解码" reading notes
 *
 * Conventions shared by every entry point
 *   - Every pointer argument named as an array is DEVICE memory unless stated otherwise,
 *     16-byte aligned, row-major and contiguous. Descriptors (gdn_dims_t,
 *     gdn_deltalog_pool_t) and `bytes` out-parameters are HOST memory.
 *   - Token-major packed layout [1, tokens, H, d] with the batch dimension dropped
 *     ([LA-Infra] "KDA实现逻辑概述" / "vLLM中Decode的实现"): q, k are [T, H, d_k]; v, o are
 *     [T, H, d_v]. Variable-length sequences are concatenated along T and delimited by
 *     cu_seqlens (device int32 [n_seqs + 1], cu_seqlens[0] = 0, non-decreasing,
 *     cu_seqlens[n_seqs] = total_tokens).
 *   - State orientation: S is d_k x d_v (row = key channel), read-out o = S^T q
 *     ([Handbook] "同一个计算的两种写法"; [DeltaLog] §1.1). State pools are
 *     [n_slots, H, d_k, d_v] fp32 and are addressed through a per-sequence/per-request slot
 *     index, like a block table ([Handbook] "投机解码与 PD 分离"; [LA-Infra] "推测解码").
 *   - q/k/v/o element type is gdn_dims_t.dtype (fp32 or bf16); the forget gate is passed
 *     as its logarithm g = log(alpha) <= 0 (fp32; [LA-Infra] "完整计算顺序" uses the log gate
 *     g_i = ln alpha_i), the write gate beta in [0, 1] (fp32). Any finite g <= 0 is
 *     accepted, per token and (per-key gate) per channel, however strong the cumulative
 *     decay within a chunk: exponentials are only ever formed of non-positive sums, or of
 *     bounded ones where their products stay exact (-inf and NaN are not accepted; the host
 *     does not read g, so they are not rejected either). The state is always fp32
 *     ([Handbook] "练习" 2: rounding would accumulate step after step).
 *   - Supported head dims: d_k == d_v in {16, 32, 64, 128}; d_k != d_v returns
 *     GDN_ERR_UNSUPPORTED. This is a contract choice: every workload on the pages uses
 *     d_k == d_v, the kernels are specialised per head dim at compile time (value tiles,
 *     fragment counts, thread maps), and independent d_k and d_v would multiply the
 *     prefill's instantiations (and the library's build time and size) about fourfold with
 *     no change for the d_k == d_v paths. Chunk sizes: 16, 32, 64.
 *   - Ownership: the caller allocates and frees all memory, including workspaces sized by
 *     the *_workspace_bytes queries. The library allocates nothing and keeps no mutable
 *     global state, except the allocation-free prefill's per-GPU device array and the cache
 *     of its per-device addresses (gdn_prefill_chunked_noalloc); it never synchronises, and
 *     launches only on `stream` (a hipStream_t; NULL = the default stream). Calls are
 *     asynchronous: device-side faults surface at the caller's next synchronisation.
 *   - Errors: every entry point returns a gdn_status_t. Arguments are validated on the host
 *     before any launch; a call that returns an error has launched nothing and changed no
 *     memory. gdn_last_error() returns a thread-local description of the last failure.
 *     No C++ exception crosses this boundary.
 *   - Debug build (libgdn_debug.so, same kernels): every entry point that takes slot indices
 *     first copies them to the host, synchronising `stream`, and returns GDN_ERR_SHAPE if a
 *     valid slot appears twice in the call. The release library does not read device
 *     arguments on the host, so there a repeated slot is undefined behaviour.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 1

typedef enum {
    GDN_OK = 0,
    GDN_ERR_NULL = 1,        /* a required pointer is NULL                                  */
    GDN_ERR_SHAPE = 2,       /* inconsistent sizes (negative counts, n_slots < 1, ...)      */
    GDN_ERR_UNSUPPORTED = 3, /* d_k/d_v/chunk/dtype/gate/M outside the supported set         */
    GDN_ERR_ALIGN = 4,       /* a device pointer is not 16-byte aligned                      */
    GDN_ERR_WORKSPACE = 5,   /* workspace smaller than the *_workspace_bytes query           */
    GDN_ERR_LAUNCH = 6       /* the HIP runtime reported an error at launch                  */
} gdn_status_t;

enum { GDN_DTYPE_F32 = 0, GDN_DTYPE_BF16 = 1 };
enum { GDN_GATE_SCALAR = 0, GDN_GATE_PER_KEY = 1 };

/* Problem description shared by all entry points (host memory).
 *   num_heads  H >= 1 (q, k and v share H)
 *   d_k, d_v   head dims (d_k == d_v in {16, 32, 64, 128})
 *   dtype      GDN_DTYPE_F32 or GDN_DTYPE_BF16 for q, k, v, o
 *   gate       GDN_GATE_SCALAR: g is [.., H] (GDN, one forget gate per head,
 *                [LA-Infra] "GDN：增加遗忘门");
 *              GDN_GATE_PER_KEY: g is [.., H, d_k] (KDA-style, one gate per key channel,
 *                decaying the key rows of S, [LA-Infra] "KDA: By Channel的遗忘门")
 *   scale      read-out scale s (o = s * S^T q; [LA-Infra] "KDA实现逻辑概述" uses
 *              head_dim^{-1/2})
 *   qk_l2norm  1: q and k are L2-normalised in fp32 inside the kernel along the head dim,
 *              x / sqrt(x.x + 1e-6) ([LA-Infra] App. 2 "为什么要L2 Norm"; the pages give an
 *              epsilon guard without a value); 0: q and k are used as given. */
typedef struct {
    int32_t num_heads;
    int32_t d_k;
    int32_t d_v;
    int32_t dtype;
    int32_t gate;
    float scale;
    int32_t qk_l2norm;
} gdn_dims_t;

/* ------------------------------------------------------------------------------ prefill */

/* Workspace needed by gdn_prefill_chunked for this problem (host computation only).
 * *bytes receives the size; returns GDN_OK or a validation error. */
int gdn_prefill_workspace_bytes(const gdn_dims_t* dims, int32_t n_seqs, int32_t total_tokens,
                                int32_t chunk, size_t* bytes);

/* Chunk-parallel prefill of packed variable-length sequences.
 * Computes, for every sequence n and head h, exactly the recurrence above over the
 * sequence's tokens, using the chunk-wise rewrite of [LA-Infra] "Prefill中的Chunk微观并行"
 * (sub-sections 计算 Δchunk / 计算 Transitionchunk / 块内输出 / 完整计算顺序): in-chunk
 * cumulative log gate, A and M from C x C products (per-key gates: 16 x 16 sub-blocks with a
 * reference point, diagonal sub-blocks computed directly when their decay is too strong for
 * the split, [LA-Infra] "附1. chunk内 A和M 的计算"), R = (I + A)^{-1} by a blocked
 * triangular solve, U = R diag(beta) V, W = R diag(beta) K_in, then the sequential pass over
 * chunks E = U - W S, O = Q_in S + M E, S <- Diag(e^{G_C}) S + K_g^T E. Chunks restart at
 * every sequence boundary; the last chunk of a sequence may be short. Splitting a sequence
 * over several calls and handing the state over through the pool gives the one-shot result
 * up to rounding ([Handbook] "同一个计算的两种写法", "在真实模型上核对"). When the call has few (sequence,
 * head) units (bf16 or fp32, d_k = d_v = 64 or 128, chunk 64, 2 x units x d_v / 16 <= the device's
 * CU count, at least 40 chunks per sequence on average), each sequence of n >= 40 chunks is
 * scanned as segments at once (two below 80 chunks, then min(K, n / 20), K = CU count /
 * (units x d_v / 16) capped at 8), composed through their transitions,
 * S_end = Transition S_start + Delta
 * ([LA-Infra] "Linear Attention Chunk-Wise"); the results then agree with the one-segment
 * pass to rounding, not bit for bit, and the workspace query includes the sections this
 * needs.
 *
 *   q, k         [total_tokens, H, d_k] dtype (device)
 *   v            [total_tokens, H, d_v] dtype (device)
 *   g            [total_tokens, H] (scalar gate) or [total_tokens, H, d_k] (per key) fp32
 *   beta         [total_tokens, H] fp32
 *   cu_seqlens   [n_seqs + 1] int32 (device)
 *   chunk        16, 32 or 64
 *   state_pool   [n_slots, H, d_k, d_v] fp32, read (initial state) and written (final state)
 *   slots        [n_seqs] int32 (device): pool slot of each sequence. A slot outside
 *                [0, n_slots) means "no slot": zero initial state, final state not stored,
 *                outputs still computed. Valid slots must be distinct within one call.
 *   has_init     [n_seqs] int32 (device) or NULL: nonzero = start from pool[slot];
 *                zero / NULL = start from the zero state.
 *   o            [total_tokens, H, d_v] dtype (device), written
 *   workspace    device scratch of at least gdn_prefill_workspace_bytes(...) bytes
 * n_seqs == 0 is a valid no-op. A sequence with no tokens leaves its final state equal to
 * its initial state (pool[slot] with has_init, else zero), which is stored in its slot. */
int gdn_prefill_chunked(const gdn_dims_t* dims, const void* q, const void* k, const void* v,
                        const float* g, const float* beta, const int32_t* cu_seqlens,
                        int32_t n_seqs, int32_t total_tokens, int32_t chunk,
                        float* state_pool, int32_t n_slots, const int32_t* slots,
                        const int32_t* has_init, void* o, void* workspace, size_t ws_bytes,
                        void* stream);

/* Chunked prefill that also exports intermediate states ("internal checkpoints").
 * A prefix cache can only resume a linear-attention layer where a state was saved, and
 * saving one at every block boundary costs a full d_k x d_v write each time, so engines ask
 * for states at a few chosen token offsets only. One forward then covers the whole prompt
 * and the kernel writes the state at those offsets into slots reserved for them
 * ([LA-Infra] "Linear Attention的Prefix Cache", part "S 到底存几份？": a backend with an
 * internal checkpoint runs [0, 2000) in one step and exports S@1920 or S@1984 on the way;
 * the offset from the step's first token must be a multiple of the kernel's chunk size).
 * Arguments and results are those of gdn_prefill_chunked, plus:
 *   ckpt_cu     [n_seqs + 1] int32 (device): the checkpoints of sequence n are entries
 *               ckpt_cu[n] .. ckpt_cu[n + 1] - 1 (ckpt_cu[0] = 0, non-decreasing,
 *               ckpt_cu[n_seqs] = n_ckpt)
 *   ckpt_pos    [n_ckpt] int32 (device): token offset p within the sequence (counted from its
 *               first token in this call); the state after the sequence's first p tokens,
 *               starting from its initial state, is exported. An offset is usable when
 *               0 < p <= length and (p % chunk == 0 or p == length). Entry i is stored iff
 *               its offset is usable and no earlier entry of the same sequence has a larger
 *               offset (entries with equal offsets all receive the state); any other entry
 *               is skipped and writes nothing.
 *   ckpt_slots  [n_ckpt] int32 (device): pool slot receiving the exported state (fp32,
 *               [H, d_k, d_v], all heads); a slot outside [0, n_slots) skips the entry (a
 *               null block). Checkpoint slots must be distinct from each other and from the
 *               `slots` of this call (the writes of one launch are not ordered).
 *   n_ckpt      number of entries (>= 0). With n_ckpt == 0 the three arrays may be NULL and
 *               the call equals gdn_prefill_chunked.
 * With checkpoints the scan runs every sequence in one segment. The exported state is then
 * bit-identical to the final state of a gdn_prefill_chunked call over the same p tokens with
 * the same chunk size, and the outputs and final states to those of gdn_prefill_chunked,
 * wherever that call also runs in one segment; where it cuts a sequence into segments (few
 * (sequence, head) units and long sequences, see gdn_prefill_chunked) the two agree to
 * rounding, not bit for bit. */
int gdn_prefill_chunked_ckpt(const gdn_dims_t* dims, const void* q, const void* k,
                             const void* v, const float* g, const float* beta,
                             const int32_t* cu_seqlens, int32_t n_seqs, int32_t total_tokens,
                             int32_t chunk, float* state_pool, int32_t n_slots,
                             const int32_t* slots, const int32_t* has_init,
                             const int32_t* ckpt_cu, const int32_t* ckpt_pos,
                             const int32_t* ckpt_slots, int32_t n_ckpt, void* o,
                             void* workspace, size_t ws_bytes, void* stream);

/* Chunked prefill that takes the raw q|k|v projection and applies the causal short
 * convolution and SiLU ([LA-Infra] "去掉分母引入卷积") while loading it, so q, k and v never
 * go to memory; everything after is gdn_prefill_chunked. For sequence n, head h, channel c
 * of plane p (q, k, v), token t of the sequence and W = conv_width:
 *   q|k|v[t, h, c] = SiLU(sum_{j<W} w[ch, j] x[t - (W-1) + j, ch]),  ch = p H d + h d + c,
 * accumulated in fp32 from the oldest tap and rounded to dtype: the values
 * gdn_conv1d_silu(planes = 3) writes, bit for bit. The outputs and states are those of
 * gdn_prefill_chunked on its three planes bit for bit with a per-key gate, or when the
 * call has few enough (sequence, head) pairs that its scan runs 16-column value tiles;
 * otherwise, with a scalar gate, gdn_prefill_chunked multiplies the given q itself and
 * scales each output row afterwards, and the two agree to rounding. A token
 * before the sequence start is the slot's conv history conv_state[slot, ch, W-1-m] (m tokens
 * before the start, m <= W-1) when conv_state is given and has_init[n] is nonzero, else 0.
 * After the call, conv_state[slot] (when given, for valid slots) holds the last W-1 inputs
 * of the sequence before the convolution, column 0 the oldest, taking inputs from before
 * the start from the old history or zero: the layout gdn_decode_fused reads and advances,
 * so a prefill followed by fused decode steps continues the sequence ([LA-Infra]
 * "vLLM中Decode的实现": one conv-state pool over the concatenated channels).
 *   x            [total_tokens, 3 H d_k] dtype (device), 16-byte aligned
 *   conv_w       [3 H d_k, conv_width] fp32 (device); conv_width 2, 3 or 4
 *   conv_state   [n_slots, 3 H d_k, conv_width - 1] dtype (device) or NULL (zero history,
 *                nothing stored); addressed by the same slot as state_pool
 *   g, beta, cu_seqlens, chunk, state_pool, slots, has_init, o, workspace: as
 *   gdn_prefill_chunked, whose workspace query applies (d_k == d_v). q, k and v are not
 *   passed. With zero tokens the conv states still advance (unchanged with history, zeroed
 *   without). */
int gdn_prefill_chunked_conv(const gdn_dims_t* dims, const void* x, const float* conv_w,
                             int32_t conv_width, void* conv_state, const float* g,
                             const float* beta, const int32_t* cu_seqlens, int32_t n_seqs,
                             int32_t total_tokens, int32_t chunk, float* state_pool,
                             int32_t n_slots, const int32_t* slots, const int32_t* has_init,
                             void* o, void* workspace, size_t ws_bytes, void* stream);

/* Allocation-free chunked prefill, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, computation and results as gdn_prefill_chunked, without the workspace
 * arguments: the workspace is a file-scope device array of GDN_NOALLOC_SCRATCH_BYTES bytes
 * inside the library, one copy per GPU, which that GPU holds from the library's first use on
 * it until the process ends. The call allocates nothing (no hipMalloc / hipFree, no
 * allocating library routine).
 *   - A call whose gdn_prefill_workspace_bytes(...) exceeds GDN_NOALLOC_SCRATCH_BYTES returns
 *     GDN_ERR_WORKSPACE before any launch (split it into several calls with the state handed
 *     over through the pool, or use gdn_prefill_chunked).
 *   - `stream` must belong to the current device (GDN_ERR_UNSUPPORTED otherwise): the
 *     array's address is resolved for the current device.
 *   - Every call on one GPU shares that GPU's array. Calls ordered on one stream are safe;
 *     calls that overlap on one GPU (different streams, or threads without ordering) race
 *     and give undefined results. The array keeps the last call's contents, which carry no
 *     meaning: nothing in it has to start at zero. */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int gdn_prefill_chunked_noalloc(const gdn_dims_t* dims, const void* q, const void* k,
                                const void* v, const float* g, const float* beta,
                                const int32_t* cu_seqlens, int32_t n_seqs,
                                int32_t total_tokens, int32_t chunk, float* state_pool,
                                int32_t n_slots, const int32_t* slots, const int32_t* has_init,
                                void* o, void* stream);

/* ------------------------------------------------------------------------------- decode */

/* One recurrent step for a batch of requests, one token each, states read and written in
 * place in a slot-indexed pool ([LA-Infra] "KDA实现逻辑概述" step list; [Handbook]
 * "投机解码与 PD 分离": each request owns a fixed slot and the batched kernel reads and
 * writes by slot index). Per request b and head h:
 *   Sbar = Diag(e^{g}) S;  vhat = Sbar^T k;  r = beta (v - vhat);
 *   S <- Sbar + k r^T;     o = scale * S^T q.
 *   q, k       [batch, H, d_k] dtype;  v, o [batch, H, d_v] dtype
 *   g          [batch, H] or [batch, H, d_k] fp32;  beta [batch, H] fp32
 *   state_pool [n_slots, H, d_k, d_v] fp32, updated in place
 *   slots      [batch] int32 (device). A slot outside [0, n_slots) marks an inactive
 *              (padding) row: its state is not touched and its o row is written as zeros.
 *              Valid slots must be distinct within one call.
 * batch == 0 is a valid no-op. */
int gdn_decode_step(const gdn_dims_t* dims, const void* q, const void* k, const void* v,
                    const float* g, const float* beta, float* state_pool, int32_t n_slots,
                    const int32_t* slots, int32_t batch, void* o, void* stream);

/* Largest number of tokens per request in one gdn_decode_spec call. */
#define GDN_SPEC_MAX_POS 16

/* Verify step of speculative decoding: every request feeds n_pos tokens (the last confirmed
 * token and n_pos - 1 draft tokens) through the recurrence of gdn_decode_step, and the state
 * after each position is kept in a slot of its own, so that after verification the next
 * round can continue from the state of the last accepted position by choosing its slot
 * instead of copying it back ([LA-Infra] "推测解码：验证后如何恢复状态": one slot per
 * candidate position in a [requests, 1 + num_spec] index table, the next round reading
 * state_pool[table[r, num_accepted - 1]]; [Handbook] "投机解码与 PD 分离").
 * Per request b and head h, with c = num_accepted[b] - 1:
 *   S = pool[spec_slots[b, c]];
 *   for j = 0 .. n_pos - 1:  S <- step(S, token (b, j));  o[b, j] = scale S^T q_{b,j};
 *                            pool[spec_slots[b, j]] = S.
 *   q, k        [batch, n_pos, H, d_k] dtype;  v, o [batch, n_pos, H, d_v] dtype
 *   g           [batch, n_pos, H] or [batch, n_pos, H, d_k] fp32;  beta [batch, n_pos, H] fp32
 *   state_pool  [n_slots, H, d_k, d_v] fp32
 *   spec_slots  [batch, n_pos] int32 (device): the request's slot for each position. A slot
 *               outside [0, n_slots) at position j means "do not keep this state" (the
 *               position is still computed). Valid slots must be distinct within one call;
 *               the starting slot spec_slots[b, c] is among them and is read before it is
 *               overwritten at position c.
 *   num_accepted [batch] int32 (device): 1 + the number of draft tokens accepted in the
 *               previous round (1 for a request that just left prefill, its state in
 *               spec_slots[b, 0]). A request whose c is outside [0, n_pos), or whose starting
 *               slot is outside [0, n_slots), is inactive: its outputs are zeros and no
 *               state is read or written.
 *   n_pos       1 .. GDN_SPEC_MAX_POS (GDN_ERR_UNSUPPORTED otherwise)
 * batch == 0 is a valid no-op. With n_pos == 1 and num_accepted == 1 the call computes
 * exactly what gdn_decode_step computes, bit for bit. */
int gdn_decode_spec(const gdn_dims_t* dims, const void* q, const void* k, const void* v,
                    const float* g, const float* beta, float* state_pool, int32_t n_slots,
                    const int32_t* spec_slots, const int32_t* num_accepted, int32_t batch,
                    int32_t n_pos, void* o, void* stream);

/* Fused KDA decode step: short-convolution update, in-kernel gates, L2 norm and the per-key
 * recurrence in one launch ([LA-Infra] "KDA实现逻辑概述" gate formulas and step list;
 * "vLLM中Decode的实现": one convolution over the concatenated q|k|v channels reading and
 * writing a conv-state pool, gates formed inside the decode kernel, q/k L2 norm in the
 * kernel; "去掉分母引入卷积": the conv state keeps the conv_width - 1 most recent inputs
 * before the convolution, [slots, 3 H d, conv_width - 1], and the output is not stored).
 * Per request b (slot s = slots[b]), head h, key channel c, with W = conv_width:
 *   for each of the 3 d channels ch of head h in the q, k, v planes:
 *     y[ch] = SiLU(sum_{j<W-1} conv_state[s, ch, j] w[ch, j] + x[b, ch] w[ch, W-1]);
 *     conv_state[s, ch, :] <- (conv_state[s, ch, 1:], x[b, ch])   (column 0 is the oldest)
 *   forget_log[c] = lower_bound * sigmoid(e^{A_log[h]} (forget_b[b, h, c] + dt_bias[h, c]))
 *   beta          = sigmoid(write_logit[b, h])
 *   then gdn_decode_step with the per-key gate g = forget_log on (q, k, v) = y of the three
 *   planes (q, k L2-normalised when dims.qk_l2norm = 1, as the page's KDA does).
 *   dims         gate must be GDN_GATE_PER_KEY (GDN_ERR_UNSUPPORTED otherwise)
 *   x            [batch, 3 H d_k] dtype: q | k | v channels before the convolution
 *   conv_w       [3 H d_k, conv_width] fp32 (column conv_width - 1 weighs the current input)
 *   conv_width   2, 3 or 4
 *   conv_state   [n_slots, 3 H d_k, conv_width - 1] dtype, read and updated in place
 *   forget_b     [batch, H, d_k] fp32;  write_logit [batch, H] fp32
 *   A_log        [H] fp32;  dt_bias [H, d_k] fp32;  lower_bound < 0 (finite; e.g. -5)
 *   state_pool   [n_slots, H, d_k, d_v] fp32;  slots [batch] int32 (device)
 *   o            [batch, H, d_v] dtype
 * Both pools are addressed by the same slot. A slot outside [0, n_slots) marks an inactive
 * row: o is zeroed and neither pool is touched. Valid slots must be distinct. batch == 0 is
 * a valid no-op. */
int gdn_decode_fused(const gdn_dims_t* dims, const void* x, const float* conv_w,
                     int32_t conv_width, void* conv_state, const float* forget_b,
                     const float* write_logit, const float* A_log, const float* dt_bias,
                     float lower_bound, float* state_pool, int32_t n_slots,
                     const int32_t* slots, int32_t batch, void* o, void* stream);

/* ----------------------------------------------------------------------------- DeltaLog */

/* DeltaLog state pool ([DeltaLog] §2.1 symbol table). All arrays are device memory:
 *   base    [n_slots, H, d_k, d_v] fp32   dense base Sbar (the dense decode pool layout)
 *   lbar    [n_slots, H, d_l] fp32        log-decay accumulated since the last merge
 *   klog    [n_slots, H, M-1, d_k] bf16   logged keys a_i (raw bf16 bit patterns)
 *   ulog    [n_slots, H, M-1, d_v] fp32   logged corrected updates b_i = beta (v - vhat)
 *   lamlog  [n_slots, H, M-1, d_l] fp32   lbar snapshot at insertion (Lambda_i)
 *   len     [n_slots, H] int32            current log length L, 0 <= L <= M-1
 *   M       merge interval (log capacity M-1), 2 <= M <= 17
 * d_l = 1 with GDN_GATE_SCALAR (one decay per head); d_l = d_k with GDN_GATE_PER_KEY
 * (KDA-style: lbar and every Lambda_i hold one log-decay per key channel, and D(x) below is
 * diag(e^x) over the key rows; [DeltaLog] §2.7, the KDA row). The gate kind of every call on
 * a pool must match the layout it was created with. Precisions follow [DeltaLog] §2.7
 * (K bf16, U, Lambda, lbar and the base fp32). */
typedef struct {
    float* base;
    float* lbar;
    uint16_t* klog;
    float* ulog;
    float* lamlog;
    int32_t* len;
    int32_t M;
} gdn_deltalog_pool_t;

/* Scratch needed by gdn_decode_deltalog (host computation). The current kernels compute
 * the key-side replay coefficients inside each workgroup and need none: *bytes = 0. */
int gdn_deltalog_workspace_bytes(const gdn_dims_t* dims, int32_t batch, int32_t M,
                                 size_t* bytes);

/* One DeltaLog decode step ([DeltaLog] §2.3 Algorithm 1, Eqs. 4-7; reads from base + log
 * per §2.4). Per request b and head h with L = len on entry and lbar' = lbar + g:
 *   vhat = (k * e^{lbar'})^T Sbar + sum_{i<L} [k^T D(lbar' - Lambda_i) K_i] U_i
 *   b    = beta (v - vhat)          (the read is against the decayed state; [LA-Infra]
 *                                     "GDN：增加遗忘门" decays before correcting)
 *   o    = scale * [(q * e^{lbar'})^T Sbar + sum_i [q^T D(lbar' - Lambda_i) K_i] U_i + (k.q) b]
 *   L <  M-1 (append): K_L = bf16(k), U_L = b, Lambda_L = lbar', L += 1, lbar = lbar'
 *   L == M-1 (merge, Eq. 6): Sbar = D(lbar') Sbar + sum_i D(lbar' - Lambda_i) K_i U_i^T
 *                             + k b^T;  lbar = 0;  L = 0.
 * The logical state after every step equals the dense decode state (Eq. 7) up to the bf16
 * rounding of logged keys. Slots, layouts and inactive rows as gdn_decode_step. Both gate
 * kinds are supported (g is [batch, H] or [batch, H, d_k]; the pool layout must match).
 * ws may be NULL when ws_bytes is 0. */
int gdn_decode_deltalog(const gdn_dims_t* dims, const void* q, const void* k, const void* v,
                        const float* g, const float* beta, const gdn_deltalog_pool_t* pool,
                        int32_t n_slots, const int32_t* slots, int32_t batch, void* o,
                        void* ws, size_t ws_bytes, void* stream);

/* Empty the log of the listed slots (all heads): L = 0, lbar = 0; the base is unchanged.
 * Used when a prefill has just written the base or a slot is reused ([DeltaLog] §2.8).
 * slots [n] int32 (device); entries outside [0, n_slots) are ignored. */
int gdn_deltalog_reset(const gdn_dims_t* dims, const gdn_deltalog_pool_t* pool,
                       int32_t n_slots, const int32_t* slots, int32_t n, void* stream);

/* Fold the pending log of the listed slots into the base without a new token
 * (Eq. 7 materialised): Sbar = D(lbar) Sbar + sum_{i<L} D(lbar - Lambda_i) K_i U_i^T,
 * then lbar = 0, L = 0. Afterwards base equals the dense state. */
int gdn_deltalog_materialize(const gdn_dims_t* dims, const gdn_deltalog_pool_t* pool,
                             int32_t n_slots, const int32_t* slots, int32_t n, void* stream);

/* ------------------------------------------------------------------------------- conv1d */

/* Causal depthwise short convolution followed by SiLU ([LA-Infra] "去掉分母引入卷积":
 * per channel, output = SiLU(x_{t-3} w[c,0] + x_{t-2} w[c,1] + x_{t-1} w[c,2] + x_t w[c,3])
 * for width 4; no mixing across channels; tokens before a sequence start count as zero).
 *   x       [total_tokens, channels] dtype (device)
 *   w       [channels, width] fp32 (device), width in {2, 3, 4}
 *   y       [planes, total_tokens, channels / planes] dtype (device): channel c is written
 *           to plane c / (channels / planes). planes = 3 splits a fused q|k|v projection into
 *           three contiguous [T, H, d] tensors ([LA-Infra] "vLLM中Decode的实现": one
 *           convolution over the concatenated channels equals three separate ones).
 *   channels must be a multiple of 8 * planes. */
int gdn_conv1d_silu(const void* x, const float* w, const int32_t* cu_seqlens, int32_t n_seqs,
                    int32_t total_tokens, int32_t channels, int32_t width, int32_t planes,
                    int32_t dtype, void* y, void* stream);

/* ------------------------------------------------------------------------------ utility */

/* Static description of a status code (never NULL). */
const char* gdn_status_string(int status);

/* Thread-local description of the last failure in this thread ("" if none). */
const char* gdn_last_error(void);

/* GDN_ABI_VERSION of the loaded library. */
int gdn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
