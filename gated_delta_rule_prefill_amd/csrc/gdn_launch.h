// Host-side launch interface between the C ABI layer (gdn_api.cpp) and the kernel files.
// Arguments arrive here already validated.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

// Prefill workspace sections (all device pointers into the caller's workspace).
// Per (chunk, head) unit, with C the chunk size, CP the contraction-padded chunk length
// (C rounded up to the MFMA K step of the element type), e the element size:
//   wneg  [C][DKP]   e   -W (correction directions, negated)      row-major
//   qin   [C][DKP]   e   Q_in = s * Q * e^{G}                      row-major
// (DKP = d_k rounded up to the MFMA contraction step, zero-padded)
//   kgt   [d_k][CP]  e   K_g^T, K_g = K * e^{G_C - G}              (key-channel major)
//   mmat  [C][CP]    e   M (lower triangular incl. diagonal)        row-major; the MFMA
//                        fragments (K-step columns) that start right of a row's 16-token
//                        block are all zero, never written and never read
//   ut    [d_v][C]   f32 U (local residuals), 16-column tiles in MFMA accumulator order,
//                        when the prep forms U (PrefillArgs::u_ws; E = U - W S cancels,
//                        so U stays fp32). Otherwise the same space holds, as three
//                        sections over all units:
//     rr  [C][CP]    e   (R - I) diag(beta)  row-major fragments, only those at or left of
//                        each row's diagonal block written
//     beta [C]       f32 beta
//     vbuf [C][d_v]  e   conv-fused prefill: v after the convolution, token rows
//     qs   [C]       f32 raw-q scan (PrefillArgs::q_raw): s e^{G_i} / |q_i| per token,
//                        in place of qin
//   decay [d_k]      f32 e^{G_C} per key channel
// Segmented scan (PrefillArgs::seg = K, the most segments a sequence is cut into) only:
//   lbuf  [C][DKP]   e   outputs of the identity run of the chunk's segment (L), row-major
//                        fragments; its zero-state outputs (fp32) replace U in ut, in the
//                        same order, as U is consumed
// and per (segment boundary j = 1 .. K-1, sequence, head), boundary-major: the state at the
// start of segment j, fp32 [d_k][d_v] (smid) and as bf16 [d_v][d_k] (smidt, an MFMA B
// operand), and segment j's transition (ptrans) and zero-state final state (delta), fp32
// [d_k][d_v].
struct PrefillWs {
    int32_t* chunk_info;   // [max_chunks][4]: seq, token start, length, 0
    int32_t* seq_first;    // [n_seqs + 1] first chunk index of each sequence
    void* wneg;
    void* qin;
    void* kgt;
    void* mmat;
    void* ut;              // U in fp32, in the scan's accumulator order (when the prep forms U)
    void* rr;              // (R - I) diag(beta), fragment-major A operand   (when the scan
    float* beta;           // beta per token of the unit                      forms U; these
    void* vbuf;            // conv-fused prefill: v rows after the convolution these share
    float* qs;             // raw-q scan: per-token row factor of q              U's section)
    float* decay;
    void* lbuf;            // segmented scan only (null otherwise)
    float* smid;
    void* smidt;
    float* ptrans;
    float* delta;
    void* dump;            // scratch words that absorb stores of lanes past a sequence end
    int64_t max_chunks;
};

struct PrefillArgs {
    int dtype, gate, H, dk, dv, chunk, cp, l2norm;
    float scale;
    const void *q, *k, *v;
    const float *g, *beta;
    const int32_t* cu_seqlens;
    int n_seqs, total_tokens;
    float* state_pool;
    int n_slots;
    const int32_t* slots;
    const int32_t* has_init;
    void* o;
    // state checkpoints inside the sequences (all null / 0 = none): the entries of sequence
    // n are [ckpt_cu[n], ckpt_cu[n + 1]); entry i asks for the state after ckpt_pos[i]
    // tokens of the sequence, stored in pool slot ckpt_slots[i]
    const int32_t *ckpt_cu, *ckpt_pos, *ckpt_slots;
    int n_ckpt;
    // fused short convolution (conv_width == 0: q, k, v are given). x is the raw q|k|v
    // projection [T, 3 H d], conv_w [3 H d, conv_width] fp32; conv_state [n_slots, 3 H d,
    // conv_width - 1] in the element type holds the history of the slot's sequence (null:
    // zero history, nothing stored)
    const void* x;
    const float* conv_w;
    void* conv_state;
    int conv_width;
    // Who forms U = R diag(beta) V, chosen by the host for the whole call from the scan's
    // tile width (scan_tiles): 1 = the prep, stored in fp32 (16-column scan tiles, bound by
    // their per-chunk dependency chain, where the scan's own loads of v rows from HBM
    // stalled each chunk); 0 = the scan, from v, (R - I) diag(beta) and beta (wider tiles,
    // bound by reading the workspace: the prep then neither reads v nor writes U).
    int u_ws;
    // 1 (scalar gate, q given, the scan forms U): the scan multiplies q itself by S and
    // scales each output row by s e^{G_i} / |q_i| (the prep's qs) instead of reading Q_in,
    // which the prep then does not write. A per-key gate scales q per channel, and the
    // conv-fused prefill has no q in memory, so both keep Q_in; so do 16-column scan tiles,
    // whose chunk step is bound by operand ingest (raw q rows arrive as 16 strided pieces
    // per load instead of one contiguous fragment).
    int q_raw;
    // K >= 2: the scan cuts each long sequence into up to K segments run at once
    // (seg_segments): the first from the initial state, each later one both from zero with the
    // real U and from the identity with U = 0; a chain pass (K > 2) carries the state across
    // the segment boundaries, and a combine pass adds (identity-run outputs) x (state at the
    // segment's start) to each later segment's outputs and forms the final state. Chosen by
    // the host when the call's (sequence, head) units leave at least half of the CUs idle;
    // 0: one segment.
    int seg;
    PrefillWs ws;
};

// Value width of the scan's workgroups, in 16-column tiles: the widest that still leaves at
// least one workgroup per CU (wider tiles share each chunk's operand stream over more
// columns; narrower ones run more sequential chains at once).
inline int scan_value_tiles(int64_t units, int dv, int ncu) {
    const int64_t tiles = units * (dv / 16);
    int nvb = 1;
    while (nvb * 2 <= dv / 16 && tiles / (nvb * 2) >= ncu) nvb *= 2;
    return nvb;
}
inline int device_cu_count() {
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();
        ncu = 256;
    }
    return ncu;
}
// The scan's value-tile width for a call (in 16-column tiles), capped per element type: an
// fp32 scan at 128 columns would need more LDS than a CU has (S^T, E^T and V^T slices).
inline int scan_tiles(int dtype, int64_t units, int dv) {
    const int cap = dtype == 1 ? 8 : 4;
    const int nvb = scan_value_tiles(units, dv, device_cu_count());
    return nvb < cap ? nvb : cap;
}

// Segmented scan: bf16 or fp32, d_k = d_v = 64 or 128, C = 64, no checkpoints, and few enough (sequence,
// head) units that at least two segments' workgroups (one 16-column tile for a first
// segment, a 16-column value tile beside an identity tile for each later one) fit on the
// chip at once; sequences long enough on average to split (SEG_MIN_CHUNKS, the length below
// which a sequence stays in one piece, as the device decides per sequence: below ~32-48
// chunks the combine pass cost more than the shorter chain saved, measured on one sequence
// at H = 4, 8 and 16). At most 64 sequences: the combine and chain passes keep their chunk
// ranges in one wave. Returns K, the most segments a sequence may be cut into (as many as
// the CUs hold, at most SEG_MAX, and no more than a sequence of all total_tokens would
// take: a K above what any sequence reaches would only add an empty chain launch), or 0.
constexpr int SEG_MIN_CHUNKS = 40;
constexpr int SEG_MAX = 8;
// Segments of a sequence of n chunks: one below SEG_MIN_CHUNKS, two below SEG_MULTI_CHUNKS,
// then min(K, n / SEG_PER_CHUNKS). Each segment past the second adds a step to the chain
// pass (~2.6 µs, bound by its fp32 products); measured on one sequence at H = 1-4, three
// segments at 64 chunks ran ~1.5 µs slower than two, four at 96 chunks 2-4 µs faster, and
// six at 128 chunks 9-10 µs faster.
constexpr int SEG_MULTI_CHUNKS = 80;
constexpr int SEG_PER_CHUNKS = 20;
__host__ __device__ inline int seg_count(int n, int kmax) {
    if (n < SEG_MIN_CHUNKS || kmax < 2) return 1;
    if (n < SEG_MULTI_CHUNKS) return 2;
    const int k = n / SEG_PER_CHUNKS;
    return k < kmax ? k : kmax;
}
inline int seg_segments(int dtype, int H, int dk, int dv, int chunk, int n_seqs,
                        int64_t total_tokens) {
    const int64_t units = (int64_t)n_seqs * H;
    if (!((dtype == 0 || dtype == 1) && dk == dv && (dk == 64 || dk == 128) && chunk == 64 &&
          units > 0 && n_seqs <= 64 && total_tokens >= (int64_t)n_seqs * SEG_MIN_CHUNKS * chunk))
        return 0;
    const int64_t k = device_cu_count() / (units * (dv / 16));
    if (k < 2) return 0;
    const int64_t longest = (total_tokens + chunk - 1) / chunk;  // chunks, at most
    return seg_count(longest < SEG_MAX * SEG_PER_CHUNKS ? (int)longest : SEG_MAX * SEG_PER_CHUNKS,
                     k < SEG_MAX ? (int)k : SEG_MAX);
}
// First segment's share of a sequence cut into k segments, in 64ths. A first-segment
// workgroup (one tile) runs a chunk faster than a later segment's (two tiles); with the
// measured two-segment optimum of 35 / 64 (the 8192-token, 16-head call; 34 to 37 were
// within noise), a later chunk costs 35 / 29 of a first one, and the share
// 35 / (35 + 29 (k - 1)) lets all k segments end together: k = 2..8 -> 35, 24, 18, 15, 12,
// 11, 9.
__host__ __device__ inline int seg_first_64(int k) {
    const int d = 29 * k + 6;
    return (2240 + d / 2) / d;
}
// First chunk of segment j (0 <= j <= k) of a sequence's chunks [c0, c1) cut into k: the
// first segment takes seg_first_64(k) / 64 of them (rounded up), the others share the rest
// evenly (j = k: c1).
__host__ __device__ inline int seg_bound(int c0, int c1, int j, int k) {
    if (j <= 0) return c0;
    if (j >= k) return c1;
    const int b1 = c0 + ((c1 - c0) * seg_first_64(k) + 63) / 64;
    return b1 + (j - 1) * (c1 - b1) / (k - 1);
}

// Chunk length / key dim rounded up to the MFMA contraction step of the element type
// (bf16: 32, fp32: 4); the padding is zero-filled.
inline int prefill_cp(int dtype, int chunk) {
    int kb = dtype == 1 ? 32 : 4;
    return ((chunk + kb - 1) / kb) * kb;
}
inline int prefill_dkp(int dtype, int dk) { return prefill_cp(dtype, dk); }

// Byte size of the prefill workspace and, if base != nullptr, its carving.
size_t prefill_ws_layout(int dtype, int H, int dk, int dv, int chunk, int n_seqs,
                         int total_tokens, void* base, PrefillWs* out);

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

struct DecodeArgs {
    int dtype, gate, H, dk, dv, l2norm;
    float scale;
    const void *q, *k, *v;
    const float *g, *beta;
    float* pool;
    int n_slots;
    const int32_t* slots;  // [batch] (one token), or [batch][n_pos] (verify step)
    int batch;
    void* o;
    // verify step of speculative decoding (null / 1 for the one-token step): n_pos tokens
    // per request, the initial state read from slots[b][num_accepted[b] - 1]
    const int32_t* num_accepted;
    int n_pos;
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

// Fused KDA decode step: short-convolution update from a conv-state pool, in-kernel gates,
// then the per-key recurrence (q, k L2-normalised when l2norm is set).
struct FusedDecodeArgs {
    int dtype, H, dk, dv, l2norm, width;
    float scale, lower_bound;
    const void* x;            // [batch][3 H d_k] q|k|v before the convolution
    const float* conv_w;      // [3 H d_k][width]
    void* conv_state;         // [n_slots][3 H d_k][width - 1], element type of x
    const float* forget_b;    // [batch][H][d_k]
    const float* write_logit; // [batch][H]
    const float* A_log;       // [H]
    const float* dt_bias;     // [H][d_k]
    float* pool;
    int n_slots;
    const int32_t* slots;
    int batch;
    void* o;
};
hipError_t launch_fused_decode(const FusedDecodeArgs& a, hipStream_t stream);

struct DeltaLogArgs {
    int dtype, gate, H, dk, dv, l2norm, M;  // gate 1: lbar and Lambda are d_k wide
    float scale;
    const void *q, *k, *v;
    const float *g, *beta;
    float* base;
    float* lbar;
    uint16_t* klog;
    float* ulog;
    float* lamlog;
    int32_t* len;
    int n_slots;
    const int32_t* slots;
    int batch;
    void* o;
};
hipError_t launch_deltalog(const DeltaLogArgs& a, hipStream_t stream);
// mode 0: reset (L = 0, lbar = 0); mode 1: materialize (fold the log into the base)
hipError_t launch_deltalog_maint(const DeltaLogArgs& a, int mode, hipStream_t stream);

struct ConvArgs {
    int dtype, channels, width, planes, n_seqs, total_tokens;
    const void* x;
    const float* w;
    const int32_t* cu_seqlens;
    void* y;
};
hipError_t launch_conv1d(const ConvArgs& a, hipStream_t stream);

// After a conv-fused prefill: conv_state[slots[n]] <- the last width-1 rows of sequence n's
// raw projection, taking the rows before its start from the old history (has_init) or zero.
hipError_t launch_conv_state_update(const PrefillArgs& a, hipStream_t stream);

}  // namespace gdn
