// Chunk-parallel prefill kernels (templates; instantiated per element type in
// prefill_bf16.hip / prefill_f32.hip).
//
// Page: [LA-Infra] "深度解析线性注意力机制演进与 AI Infra 实现", section "Prefill中的Chunk微观并行":
//   "计算 Δchunk"        local residuals U from the unit lower-triangular system (I + A) U = B V,
//   "计算 Transitionchunk" correction directions W from (I + A) W = B K_in with the same R,
//   "块内输出"            O = Q_in S_0 + M E without materialising per-token states,
//   "完整计算顺序"         the six-step order (G, K_in/K_g/e^{G_C}, A and R, U and W, E and S_C,
//                        Q_in/M/O); the blocked inverse of L = I + A through 2x2 blocks
//                        ((L^{-1})_{21} = -L_22^{-1} L_21 L_11^{-1}) with 16x16 leaves;
// appendix "附1. chunk内 A和M 的计算" (per-key gates: 16x16 sub-blocks, reference point = the
// first token of the row block, A and M from one pass sharing the key-side operand).
// Orientation: S is d_k x d_v here (the page's S^T); the page's E^T K_g is K_g^T E.
//
// Work split on MI355X:
//   prep  (grid: chunks x heads, fully parallel): everything that depends only on the chunk
//         — G, A and M on MFMA, R by blocked substitution in fp32, W on MFMA — written once
//         to a workspace in MFMA-operand-ready layouts (-W and Q_in row-major, K_g^T
//         key-major, M row-major, e^{G_C}); U = R diag(beta) V either on MFMA here (fp32,
//         in the scan's accumulator order) or, for the scan's wider value tiles, by the
//         scan itself from v, with (R - I) diag(beta) and beta from the prep.
//   scan  (grid: sequences x heads x d_v/16 value tiles, serial over a sequence's chunks):
//         the only sequential part. A 16- to 128-column slice of the fp32 state lives in
//         MFMA accumulators across the whole sequence; per chunk
//           E = U - W S,  O = Q_in S + M E,  S <- Diag(e^{G_C}) S + K_g^T E
//         with E and O rows on separate waves and each wave's operands of the next chunk
//         prefetched into its registers during the current one.
//         The value tiles of one (sequence, head) are placed on the same XCD so the shared
//         per-chunk operands are served from that XCD's L2.
#pragma once
#include <algorithm>
#include <climits>
#include <type_traits>

#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {

constexpr int PF_THREADS = 256;
constexpr int PF_WAVES = PF_THREADS / WAVE;
constexpr int SCAN_BV = 16;

template <typename T, int DK, int DV, int C>
struct PfCfg {
    using MM = Mma<T>;
    static constexpr int KB = MM::KB;
    static constexpr int KPL = MM::KPL;
    static constexpr int CP = ((C + KB - 1) / KB) * KB;     // padded token contraction
    static constexpr int DKP = ((DK + KB - 1) / KB) * KB;   // padded key-channel contraction
    static constexpr int PADE = 16 / (int)sizeof(T);          // 16-byte row padding
    static constexpr int LDK = DKP + PADE;                    // LDS row stride, d_k rows
    static constexpr int LDC = CP + PADE;                     // LDS row stride, token rows
    static constexpr int NB = C / 16;                         // 16-token blocks
};

// chunk -> (sequence, first token, length) from the per-sequence first-chunk table
struct ChunkLoc {
    int seq, tok0, len;
};

// Up to one wave's worth of sequences, every wave forms the first-chunk table itself: lane n
// holds the exclusive and inclusive prefix sums of ceil(len_s / C) at sequence n (the same
// table the separate seq_first pass writes for longer lists), so no extra launch runs.
constexpr int SEQ_INLINE_MAX = WAVE;
struct WaveSeqTable {
    int excl, incl;
};
__device__ __forceinline__ WaveSeqTable wave_seq_table(const int32_t* cu, int n_seqs, int C) {
    const int l = lane_id();
    int cnt = 0;
    if (l < n_seqs) cnt = (max(0, cu[l + 1] - cu[l]) + C - 1) / C;
    int x = cnt;
#pragma unroll
    for (int off = 1; off < WAVE; off <<= 1) {
        const int y = __shfl_up(x, off, WAVE);
        if (l >= off) x += y;
    }
    return {x - cnt, x};
}
__device__ __forceinline__ ChunkLoc locate_chunk_inline(int c, const int32_t* cu, int n_seqs,
                                                        int C, int total_tokens) {
    ChunkLoc r;
    r.seq = -1;
    r.tok0 = 0;
    r.len = 0;
    const WaveSeqTable t = wave_seq_table(cu, n_seqs, C);
    // the one non-empty sequence whose chunk range holds c (none past the last chunk)
    const uint64_t m = __ballot(lane_id() < n_seqs && t.excl <= c && c < t.incl);
    if (m == 0) return r;
    const int n = __builtin_ctzll(m);
    const int first = __builtin_amdgcn_readlane(t.excl, n);
    r.tok0 = cu[n] + (c - first) * C;
    r.len = min(C, min(cu[n + 1], total_tokens) - r.tok0);
    if (r.tok0 < 0 || r.len <= 0) {  // inconsistent cu_seqlens: never index outside q/k/v
        r.len = 0;
        return r;
    }
    r.seq = n;
    return r;
}
__device__ __forceinline__ ChunkLoc locate_chunk(int c, const int32_t* seq_first,
                                                 const int32_t* cu, int n_seqs, int C,
                                                 int total_tokens) {
    ChunkLoc r;
    r.seq = -1;
    r.tok0 = 0;
    r.len = 0;
    if (c >= seq_first[n_seqs]) return r;
    int lo = 0, hi = n_seqs;  // find last n with seq_first[n] <= c
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (seq_first[mid] <= c) lo = mid; else hi = mid;
    }
    r.tok0 = cu[lo] + (c - seq_first[lo]) * C;
    r.len = min(C, min(cu[lo + 1], total_tokens) - r.tok0);
    if (r.tok0 < 0 || r.len <= 0) {  // inconsistent cu_seqlens: never index outside q/k/v
        r.len = 0;
        return r;
    }
    r.seq = lo;
    return r;
}

// Prep order for the two-segment scan (PrefillArgs::seg = 2): dispatch slot i of NG groups
// of 8 chunks -> the group prepared there. The scan starts each segment at its first
// chunks, so those are prepared last (the likeliest to be still cached when the scan reads
// them): the first segment's groups (the first seg_first_64(2) / 64, as the split) and the
// second's interleave in descending order, ending with group 0 and the second segment's
// first group. Same-box headline scan 61 -> 59.4 µs; one plain descending order gained
// nothing.
__device__ __forceinline__ int seg_prep_group(int i, int NG) {
    const int sg = (NG * seg_first_64(2) + 63) / 64, na = sg, nb = NG - sg, mn = min(na, nb);
    const int r = NG - 1 - i;  // 0: dispatched last
    if (r < 2 * mn) return (r % 2 == 0) ? r / 2 : sg + r / 2;
    return na > nb ? r - mn : sg + (r - mn);
}

// The same for a call cut into k > 2 segments (the groups cut as a sequence of NG groups
// would be): the slots dispatched last take, pass by pass, the m-th group of every segment
// that long, segments in order (pass 0: each segment's first group). Slot r from the end
// lies in the pass m with before(m) <= r < before(m + 1), before(m) = sum_s min(len_s, m)
// the slots of the passes ahead of it, found by bisection.
__device__ __forceinline__ int seg_prep_group_k(int i, int NG, int k) {
    int b[SEG_MAX + 1];
#pragma unroll
    for (int s = 0; s <= SEG_MAX; s++) b[s] = seg_bound(0, NG, min(s, k), k);
    auto before = [&](int m) {
        int c = 0;
#pragma unroll
        for (int s = 0; s < SEG_MAX; s++) c += min(b[s + 1] - b[s], m);  // empty past k
        return c;
    };
    const int r = NG - 1 - i;  // 0: dispatched last
    int lo = 0, hi = NG;       // before(0) = 0 <= r < NG = before(NG)
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (before(mid) <= r) lo = mid;
        else hi = mid;
    }
    int t = r - before(lo), grp = i;
#pragma unroll
    for (int s = 0; s < SEG_MAX; s++) {
        const bool has = b[s + 1] - b[s] > lo;
        if (has && t == 0) grp = b[s] + lo;
        t -= has ? 1 : 0;
    }
    return grp;
}

// Fragment-major layout of an R x K MFMA A-operand matrix (R a multiple of 16, K of KB):
// the 16 x KB fragment (row block rb, k block kb) is stored as 64 lane slots of KPL elements,
// slot `lane` holding X[16 rb + (lane & 15)][kb KB + (lane >> 4) KPL + e]. A wave then loads a
// fragment as one contiguous run (1 KiB for bf16, 8 full cache lines) instead of 16 rows that
// are each touched for 64 bytes; the vector-memory pipe of a CU processes the former at
// twice the rate.
template <typename T>
struct Frag {
    static constexpr int KB = Mma<T>::KB, KPL = Mma<T>::KPL;
    __device__ __forceinline__ static int off(int row, int col, int K) {
        const int kb = col / KB, kk = col - kb * KB;
        const int ln = (row & 15) + 16 * (kk / KPL);
        return (((row >> 4) * (K / KB) + kb) * 64 + ln) * KPL + (kk % KPL);
    }
    // N consecutive columns starting at col (col a multiple of N)
    template <int N>
    __device__ __forceinline__ static void store_run(T* base, int row, int col, int K,
                                                     const float* v) {
        if constexpr (KPL >= N) {
            if constexpr (N == 8) store8<T>(base + off(row, col, K), v);
            else store4<T>(base + off(row, col, K), v);
        } else {
#pragma unroll
            for (int i = 0; i < N; i++) base[off(row, col + i, K)] = from_f32<T>(v[i]);
        }
    }
    __device__ __forceinline__ static const T* ptr(const T* base, int rb, int kb, int K, int ln) {
        return base + ((rb * (K / KB) + kb) * 64 + ln) * KPL;
    }
};

// =====================================================================================
// prep kernel
// =====================================================================================
// One workgroup per (chunk, head); wave w owns token block w (16 tokens) for the row-wise
// work. Phases (LDS barriers between them):
//   P0  loads (K, Q, V straight into MFMA row fragments), L2 norm, gate prefix sums
//   P1  Q_in, K_g^T, (beta K_in)^T via identity-MFMA transposes; A and M tiles of the
//       wave's own row block (its key and query rows stay in registers)
//   P2  16x16 leaf inverses of I + A (forward substitution, one lane per column), V^T
//   P3  2x2 block merges on fp32 MFMA (16 -> 32 -> 64), in place over A
//   P4  -W and U on MFMA, written to the workspace
template <typename T, int DK, int DV, int C, bool PERKEY, bool CONV = false>
struct PrepSmem {
    using F = PfCfg<T, DK, DV, C>;
    // live for the whole kernel
    alignas(16) float bs[C];          // beta
    alignas(16) float eg[C];          // scalar gate: e^{G_i}
    alignas(16) float egc[C];         // scalar gate: e^{G_C - G_i}
    alignas(16) T kint[DK][F::LDC];   // (diag(beta) K_in)^T
    union {
        struct {                      // P0-P1: keys in fragment-major order, gates
            alignas(16) T ks[C * F::DKP];
            alignas(16) float gs[PERKEY ? C : 1][PERKEY ? DK + 4 : C];  // cumulative log gate
            float gseg[PERKEY ? PF_THREADS / DK : 1][PERKEY ? DK : 1];    // segment totals
        } a;
        struct {                      // from barrier #2 on
            union {
                alignas(16) float ar[C][C + 1];  // A (strictly lower), then R = (I + A)^{-1}
                                                 // in place; the strictly upper part is
                                                 // merge scratch
                alignas(16) T va[PERKEY ? 1 : DV][F::LDC];  // scalar gate: V^T (when the
                                                            // prep forms U), once R is done
            };
            alignas(16) T rs[C][F::LDC];     // R as an MFMA operand
            alignas(16) T vt[PERKEY ? DV : 1][F::LDC];  // per-key gate: V^T (prep forms U)
        } b;
    } u;
    // per-key conv: the weights, kept for V's convolution after P0 (the other members keep
    // their offsets)
    alignas(16) float cw[PERKEY && CONV ? 3 * DK * 4 : 1];
};

template <bool PERKEY, int DK, int C>
__device__ __forceinline__ float gval(const float (*gs)[PERKEY ? DK + 4 : C], int i, int c) {
    if constexpr (PERKEY) return gs[i][c];
    else return gs[0][i];
}

// Identity B fragments: MFMA(A_rows, I_h) returns, in accumulator layout, the 16 x 16 block
// of the row fragment A_rows whose columns are selected by h, i.e. lane (g, n) receives
// A[4g + e][16 cb + n] — four consecutive rows of one column, the transposed orientation.
template <typename T> struct Ident;
template <> struct Ident<bf16> {
    static constexpr int N = 2;  // 32 columns per fragment: two 16-column halves
    __device__ __forceinline__ static void make(bf16x8 (&id)[2]) {
        const int g = lane_id() >> 4, n = lane_id() & 15;
#pragma unroll
        for (int h = 0; h < 2; h++)
#pragma unroll
            for (int e = 0; e < 8; e++) id[h][e] = (bf16)((8 * g + e == 16 * h + n) ? 1.f : 0.f);
    }
    template <int NK>
    __device__ __forceinline__ static f32x4 transpose(const bf16x8 (&rows)[NK], int cb,
                                                      const bf16x8 (&id)[2]) {
        return Mma<bf16>::mma(rows[cb >> 1], id[cb & 1], zero4());
    }
};
template <> struct Ident<float> {
    static constexpr int N = 4;  // 4 columns per fragment
    __device__ __forceinline__ static void make(float (&id)[4]) {
        const int g = lane_id() >> 4, n = lane_id() & 15;
#pragma unroll
        for (int s4 = 0; s4 < 4; s4++) id[s4] = (4 * s4 + g == n) ? 1.f : 0.f;
    }
    template <int NK>
    __device__ __forceinline__ static f32x4 transpose(const float (&rows)[NK], int cb,
                                                      const float (&id)[4]) {
        f32x4 acc = zero4();
#pragma unroll
        for (int s4 = 0; s4 < 4; s4++) acc = Mma<float>::mma(rows[4 * cb + s4], id[s4], acc);
        return acc;
    }
};

// Scalar gate: V^T shares its LDS with A/R (46.6 KiB at d = 128, C = 64) and the register
// budget allows three waves per SIMD, so three workgroups share a CU and hide more of the
// load latency of each unit's q, k, v.
//
// CONV: q, k and v are formed on load from the raw projection x by the causal short
// convolution and SiLU ([LA-Infra] "去掉分母引入卷积"): each lane loads its own row of x and
// the conv taps on earlier rows reach it through a rotation inside its 16-lane row group;
// lanes 13..15 also load the three rows before the block (from the previous block, the
// previous chunk, or the sequence's conv history). The weights of the head's channels sit
// in LDS for the duration of P0.
// Occupancy floor: 3 waves per SIMD (2 with per-key gates), which fits the bf16 prep's
// registers. fp32 operands take twice the registers for the same elements: at d = 64 that
// floor made the compiler spill to scratch (2 thousand spill instructions), so fp32 at
// d = 64 asks for one wave per SIMD and the whole register file (no spills; prep 854 ->
// 205 µs at 8192 tokens x 16 heads). At d = 128 the fp32 working set exceeds even that
// (it spills either way, and more slowly with one wave), so it keeps the floor.
template <typename T, int DK>
constexpr int prep_waves_per_eu(bool perkey) {
    return sizeof(T) == 4 && DK == 64 ? 1 : (perkey ? 2 : 3);
}
template <typename T, int DK, int DV, int C, bool PERKEY, bool CONV>
__global__ __launch_bounds__(PF_THREADS)
__attribute__((amdgpu_waves_per_eu(prep_waves_per_eu<T, DK>(PERKEY)))) void prefill_prep_kernel(PrefillArgs a) {
    using F = PfCfg<T, DK, DV, C>;
    using MM = typename F::MM;
    using frag = typename MM::frag;
    constexpr int KB = F::KB, KPL = F::KPL, CP = F::CP, NB = F::NB, DKP = F::DKP;
    constexpr int NK = DKP / KB;                       // row fragments over d_k
    constexpr int NV = ((DV + KB - 1) / KB);           // row fragments over d_v
    extern __shared__ __align__(16) unsigned char smem_raw[];
    auto& sm = *reinterpret_cast<PrepSmem<T, DK, DV, C, PERKEY, CONV>*>(smem_raw);
    T (*const vt)[F::LDC] = PERKEY ? sm.u.b.vt : sm.u.b.va;
    // who forms U (uniform over the grid): the prep (fp32, into the workspace) or the scan
    const bool uws = a.u_ws != 0;

    // Unit mapping. Workgroups are dealt round-robin over the 8 XCDs (blockIdx % 8).
    // Without the convolution the heads of one chunk get consecutive ids within one XCD: a
    // token's gates and betas of all heads share a cache line, which is then fetched into
    // one L2 instead of eight (32 x 2048-token batch: prep reads 873 -> 815 MB, 445 -> 438
    // µs). The grid covers the chunk count rounded up to 8; the extra workgroups find no
    // chunk and exit. The conv-fused prep keeps chunk-major ids (chunk c, head h at
    // c H + h): its first rows read the previous chunk's last rows of the same head, which
    // that order keeps on one XCD when 8 divides H (the XCD-aware order raised the KDA
    // batch's reads by 156 MB).
    const int H = a.H;
    int c, h;
    if constexpr (CONV) {
        c = blockIdx.x / H;
        h = blockIdx.x - c * H;
    } else {
        const int xcd = blockIdx.x & 7, jj = blockIdx.x >> 3;
        int grp = jj / H;
        const int NG = (int)((a.ws.max_chunks + 7) / 8);
        if (a.seg == 2)
            grp = seg_prep_group(grp, NG);
        else if (a.seg > 2)
            grp = seg_prep_group_k(grp, NG, seg_count((int)min(a.ws.max_chunks, (int64_t)SEG_MAX * SEG_PER_CHUNKS), a.seg));
        c = grp * 8 + xcd;
        h = jj - (jj / H) * H;
    }
    // The grid may exceed the chunk bound the workspace was sized for (rounded up to 8, or
    // cu_seqlens that break the header's contract and describe more chunks): such a
    // workgroup has no workspace unit and stores nothing.
    if (c >= a.ws.max_chunks) return;
    const ChunkLoc loc =
        a.n_seqs <= SEQ_INLINE_MAX
            ? locate_chunk_inline(c, a.cu_seqlens, a.n_seqs, C, a.total_tokens)
            : locate_chunk(c, a.ws.seq_first, a.cu_seqlens, a.n_seqs, C, a.total_tokens);
    if (loc.seq < 0) return;
    const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
    const int g4 = lane >> 4, r16 = lane & 15;
    const size_t u = (size_t)c * H + h;  // (chunk, head) workspace unit
    const bool own = w < NB;             // this wave owns token block w
    const int row = w * 16 + r16;        // token row of this lane's row fragments
    const bool rvalid = own && row < loc.len;

    // ------------------------------------------------------------------------ P0 loads
    frag kf[NK], qf[NK], vf[NV];
    // conv-fused: weights (registers, then LDS), own rows and halo rows of x
    constexpr int NWL = CONV ? (3 * DK * 4 + PF_THREADS - 1) / PF_THREADS : 1;
    float wreg[NWL];
    frag xh[CONV ? 2 * NK + NV : 1];
    static_assert(!CONV || DK == DV, "the fused convolution assumes d_k == d_v");
    static_assert(!CONV || PERKEY || F::LDC * sizeof(T) >= 48,
                  "conv weights do not fit the K_in^T area");
    if constexpr (CONV) {
        const int W = a.conv_width;
        // tap d (token t - d) of channel ch of plane p at [(p DK + ch) 4 + d]; taps >= W are 0
#pragma unroll
        for (int k = 0; k < NWL; k++) {
            const int i = tid + k * PF_THREADS;
            const int p = i / (DK * 4), ch = (i >> 2) % DK, d = i & 3;
            wreg[k] = (i < 3 * DK * 4 && d < W)
                          ? a.conv_w[((size_t)(p * H + h) * DK + ch) * W + (W - 1 - d)]
                          : 0.f;
        }
        sched_fence();
        const size_t XC = (size_t)3 * H * DK;
        const T* xb = reinterpret_cast<const T*>(a.x);
        const int ss = a.cu_seqlens[loc.seq];
        const int hrow = loc.tok0 + w * 16 + r16 - 16;  // halo row of lanes 13..15
        const bool hlane = own && r16 >= 13;
        // a row past the chunk's last token feeds only padding rows: never loaded
        const bool hin = hlane && hrow >= ss && hrow >= 0 && hrow < loc.tok0 + loc.len;
        const T* xo = xb + (size_t)(loc.tok0 + row) * XC + (size_t)h * DK;
        const T* xhp = xb + (size_t)(hin ? hrow : 0) * XC + (size_t)h * DK;
#pragma unroll
        for (int f = 0; f < 2 * NK + NV; f++) {
            const int p = f < NK ? 0 : (f < 2 * NK ? 1 : 2);
            const int kb = f - p * NK;
            const int c0 = kb * KB + g4 * KPL;
            const size_t po = (size_t)p * H * DK + c0;
            frag xv = MM::zero(), hv = MM::zero();
            if (rvalid && c0 < DK) xv = MM::load(xo + po);
            if (hin && c0 < DK) hv = MM::load(xhp + po);
            if (p == 0) qf[kb] = xv;
            else if (p == 1) kf[kb] = xv;
            else vf[kb] = xv;
            xh[f] = hv;
        }
        // rows before the sequence start: the slot's conv history, if it has one
        const int slot = a.slots[loc.seq];
        const bool hist = a.conv_state != nullptr && 0 <= slot && slot < a.n_slots &&
                          a.has_init != nullptr && a.has_init[loc.seq] != 0;
        const int m = ss - hrow;  // 1..W-1 for a history row
        if (hist && hlane && m >= 1 && m <= W - 1) {
            const T* cs = reinterpret_cast<const T*>(a.conv_state) +
                          ((size_t)slot * XC + (size_t)h * DK) * (W - 1) + (W - 1 - m);
#pragma unroll
            for (int f = 0; f < 2 * NK + NV; f++) {
                const int p = f < NK ? 0 : (f < 2 * NK ? 1 : 2);
                const int c0 = (f - p * NK) * KB + g4 * KPL;
                if (c0 < DK) {
                    const T* src = cs + ((size_t)p * H * DK + c0) * (W - 1);
                    if constexpr (KPL == 1) xh[f] = src[0];
                    else {
#pragma unroll
                        for (int e = 0; e < KPL; e++) xh[f][e] = src[(size_t)e * (W - 1)];
                    }
                }
            }
        }
        sched_fence();
    } else {
        const size_t tk = ((size_t)(loc.tok0 + row) * H + h);
        const T* kg = reinterpret_cast<const T*>(a.k) + tk * DK;
        const T* qg = reinterpret_cast<const T*>(a.q) + tk * DK;
        const T* vg = reinterpret_cast<const T*>(a.v) + tk * DV;
#pragma unroll
        for (int kb = 0; kb < NK; kb++) {
            const int c0 = kb * KB + g4 * KPL;
            kf[kb] = MM::zero();
            qf[kb] = MM::zero();
            if (rvalid && c0 < DK) {
                kf[kb] = MM::load(kg + c0);
                qf[kb] = MM::load(qg + c0);
            }
        }
        // v only when the prep forms U; otherwise the scan reads it
#pragma unroll
        for (int kb = 0; kb < NV; kb++) {
            const int c0 = kb * KB + g4 * KPL;
            vf[kb] = MM::zero();
            if (uws && rvalid && c0 < DV) vf[kb] = MM::load(vg + c0);
        }
    }
    constexpr int GP = PERKEY ? PF_THREADS / DK : 1;  // per-key gate: row segments per channel
    constexpr int GR = PERKEY ? C / GP : 1;           // rows per segment
    float gv[GR];
    const int gch = tid % DK, gseg = tid / DK;
    if constexpr (PERKEY) {
#pragma unroll
        for (int r = 0; r < GR; r++) {
            const int i = gseg * GR + r;
            gv[r] = i < loc.len ? a.g[((size_t)(loc.tok0 + i) * H + h) * DK + gch] : 0.f;
        }
    }
    float gsc = 0.f, bval = 0.f;
    if (!PERKEY && w == 0)
        gsc = (lane < loc.len && lane < C) ? a.g[(size_t)(loc.tok0 + lane) * H + h] : 0.f;
    if (tid < C && tid < loc.len) bval = a.beta[(size_t)(loc.tok0 + tid) * H + h];

    // Conv weights: scalar gate in the K_in^T area (written only after barrier #1); per-key
    // gate in an area of their own, because V's convolution there runs after P0 (see below).
    float* const wl = PERKEY ? &sm.cw[0] : reinterpret_cast<float*>(&sm.kint[0][0]);
    // convolution + SiLU of fragment f (q: f < NK, k: f < 2 NK, v: the rest), in place;
    // every call sits in an unrolled loop, so f is a constant there
    auto conv_frag = [&](const int f) {
            const int p = f < NK ? 0 : (f < 2 * NK ? 1 : 2);
            const int kb = f - p * NK;
            const int c0 = kb * KB + g4 * KPL;
            frag& xf = p == 0 ? qf[kb] : (p == 1 ? kf[kb] : vf[kb]);
            if (c0 >= DK) return;  // zero padding columns stay zero
            // x at t - d (d = 1..3) arrives by rotating the row group by d: lane s sends to
            // lane (s + d) mod 16, its own row if that lane follows it, else (wrapping
            // around, s >= 16 - d) the halo row that lane needs
            const frag x1 = row_ror<1>(r16 >= 15 ? xh[f] : xf);
            const frag x2 = row_ror<2>(r16 >= 14 ? xh[f] : xf);
            const frag x3 = row_ror<3>(r16 >= 13 ? xh[f] : xf);
            frag out;
#pragma unroll
            for (int e = 0; e < KPL; e++) {
                const f32x4 wt = *reinterpret_cast<const f32x4*>(wl + (p * DK + c0 + e) * 4);
                auto el = [&](const frag& v) {
                    if constexpr (KPL == 1) return to_f32(v);
                    else return to_f32(v[e]);
                };
                // oldest tap first, as the standalone convolution accumulates; the taps a
                // narrower convolution lacks have weight 0 and add exactly +0 to the zero
                // accumulator (finite inputs)
                float acc = fmaf(wt[3], el(x3), 0.f);
                acc = fmaf(wt[2], el(x2), acc);
                acc = fmaf(wt[1], el(x1), acc);
                acc = fmaf(wt[0], el(xf), acc);
                const T y = from_f32<T>(silu_f32(acc));
                if constexpr (KPL == 1) out = y;
                else out[e] = y;
            }
            xf = rvalid ? out : MM::zero();  // rows past the chunk stay zero
    };
    // v after the convolution to the workspace, where the scan forms U from it (rows past
    // the chunk as zeros)
    auto store_vrows = [&]() {
        if (uws || !own) return;
        T* vb = reinterpret_cast<T*>(a.ws.vbuf) + (u * C + row) * DV + g4 * KPL;
#pragma unroll
        for (int kb = 0; kb < NV; kb++)
            if (kb * KB + g4 * KPL < DV) *reinterpret_cast<frag*>(vb + kb * KB) = vf[kb];
    };
    if constexpr (CONV) {
#pragma unroll
        for (int k = 0; k < NWL; k++) {
            const int i = tid + k * PF_THREADS;
            if (i < 3 * DK * 4) wl[i] = wreg[k];
        }
        lds_barrier();  // #0: conv weights in LDS
        // q and k here (the L2 norm and the key tiles need them); per-key: v later, in time
        // the waves would otherwise spend waiting at barriers #2 and #3
#pragma unroll
        for (int f = 0; f < 2 * NK + NV; f++) {
            if (!own) break;
            if (PERKEY && f >= 2 * NK) break;
            conv_frag(f);
        }
        if constexpr (!PERKEY) store_vrows();
    }

    // L2 norm of q and k rows: a row lives in the 4 lane groups sharing r16
    float iqn = 1.f;  // 1 / |q| of the lane's row (1 without the norm)
    if (a.l2norm) {
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int kb = 0; kb < NK; kb++) {
#pragma unroll
            for (int e = 0; e < KPL; e++) {
                float x, y;
                if constexpr (KPL == 1) { x = to_f32(kf[kb]); y = to_f32(qf[kb]); }
                else { x = to_f32(kf[kb][e]); y = to_f32(qf[kb][e]); }
                // explicit FMAs: every instantiation rounds the same way
                sk = fmaf(x, x, sk);
                sq = fmaf(y, y, sq);
            }
        }
        sk += __shfl_xor(sk, 16, WAVE);
        sk += __shfl_xor(sk, 32, WAVE);
        sq += __shfl_xor(sq, 16, WAVE);
        sq += __shfl_xor(sq, 32, WAVE);
        const float ik = rsqrtf(sk + 1e-6f), iq = rsqrtf(sq + 1e-6f);
        iqn = iq;
#pragma unroll
        for (int kb = 0; kb < NK; kb++) {
            if constexpr (KPL == 1) {
                kf[kb] = from_f32<T>(to_f32(kf[kb]) * ik);
                qf[kb] = from_f32<T>(to_f32(qf[kb]) * iq);
            } else {
#pragma unroll
                for (int e = 0; e < KPL; e++) {
                    kf[kb][e] = from_f32<T>(to_f32(kf[kb][e]) * ik);
                    qf[kb][e] = from_f32<T>(to_f32(qf[kb][e]) * iq);
                }
            }
        }
    }
    // keys to LDS in fragment-major order (conflict-free 16-byte accesses)
    if (own) {
#pragma unroll
        for (int kb = 0; kb < NK; kb++) {
            const int off = ((w * NK + kb) * 64 + lane) * KPL;
            *reinterpret_cast<frag*>(&sm.u.a.ks[off]) = kf[kb];
        }
    }
    if (tid < C) {
        sm.bs[tid] = bval;
        if (!uws) a.ws.beta[u * C + tid] = bval;
    }
    if constexpr (PERKEY) {
        float run = 0.f;
#pragma unroll
        for (int r = 0; r < GR; r++) {
            run += gv[r];
            gv[r] = run;
        }
        sm.u.a.gseg[gseg][gch] = run;
        lds_barrier();
        float base = 0.f;
        for (int p2 = 0; p2 < gseg; p2++) base += sm.u.a.gseg[p2][gch];
#pragma unroll
        for (int r = 0; r < GR; r++) sm.u.a.gs[gseg * GR + r][gch] = gv[r] + base;
    } else if (w == 0) {
        float x = gsc;
#pragma unroll
        for (int off = 1; off < WAVE; off <<= 1) {
            const float y = __shfl_up(x, off, WAVE);
            if (lane >= off) x += y;
        }
        const float gC = __shfl(x, C - 1, WAVE);
        if (lane < C) {
            sm.u.a.gs[0][lane] = x;
            sm.eg[lane] = __expf(x);
            sm.egc[lane] = __expf(gC - x);
        }
    }
    lds_barrier();  // #1: gates, beta, keys in LDS

    // --------------------------------------------------- P1a: own token block, row-wise
    frag idf[Ident<T>::N];
    Ident<T>::make(idf);
    if (own) {
        // Q_in = s * Q * e^{G} -> workspace (fragment-major slot of this lane); or, when the
        // scan multiplies q itself, only the row factor s e^{G_i} / |q_i|
        T* qin = reinterpret_cast<T*>(a.ws.qin) + u * C * DKP;
        const float erow = PERKEY ? 1.f : sm.eg[row];
        const bool qraw = !PERKEY && a.q_raw;
        if (qraw && g4 == 0) a.ws.qs[u * C + row] = a.scale * erow * iqn;
        if (!qraw) {
#pragma unroll
            for (int kb = 0; kb < NK; kb++) {
                float vals[KPL];
#pragma unroll
                for (int e = 0; e < KPL; e++) {
                    const int ch = kb * KB + g4 * KPL + e;
                    float qv;
                    if constexpr (KPL == 1) qv = to_f32(qf[kb]);
                    else qv = to_f32(qf[kb][e]);
                    float f = erow;
                    if constexpr (PERKEY) f = ch < DK ? __expf(sm.u.a.gs[row][ch]) : 0.f;
                    vals[e] = a.scale * qv * f;
                }
                T* dst = qin + ((w * NK + kb) * 64 + lane) * KPL;
                if constexpr (KPL == 8) store8<T>(dst, vals);
                else *dst = from_f32<T>(vals[0]);
            }
        }
        // K transposes: lane (g4, n) gets K[16w + 4 g4 + e][16 cb + n]; scaled twice into
        // (beta K_in)^T (LDS) and K_g^T (workspace, fragment-major)
        T* kgt = reinterpret_cast<T*>(a.ws.kgt) + u * DK * CP;
#pragma unroll
        for (int cb = 0; cb < DK / 16; cb++) {
            const f32x4 kt = Ident<T>::template transpose<NK>(kf, cb, idf);
            const int ch = cb * 16 + r16;
            const int t0 = w * 16 + g4 * 4;
            float kin[4], kgv[4];
            const float gC = PERKEY ? sm.u.a.gs[C - 1][ch] : 0.f;
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int t = t0 + e;
                float fin, fg;
                if constexpr (PERKEY) {
                    const float gt = sm.u.a.gs[t][ch];
                    fin = __expf(gt);
                    fg = __expf(gC - gt);
                } else {
                    fin = sm.eg[t];
                    fg = sm.egc[t];
                }
                kin[e] = sm.bs[t] * kt[e] * fin;
                kgv[e] = kt[e] * fg;
            }
            store4<T>(&sm.kint[ch][t0], kin);
            Frag<T>::template store_run<4>(kgt, ch, t0, CP, kgv);
        }
    }
    // zero the K_g^T / (beta K_in)^T token padding [C, CP)
    if constexpr (CP > C) {
        T* kgt = reinterpret_cast<T*>(a.ws.kgt) + u * DK * CP;
        for (int idx = tid; idx < DK * ((CP - C) / 4); idx += PF_THREADS) {
            const int ch = idx / ((CP - C) / 4), t0 = C + (idx % ((CP - C) / 4)) * 4;
            float z[4] = {0.f, 0.f, 0.f, 0.f};
            store4<T>(&sm.kint[ch][t0], z);
            Frag<T>::template store_run<4>(kgt, ch, t0, CP, z);
        }
    }
    // Q_in padding channels [DK, DKP) were loaded as zeros and stored above
    if (tid < DK) a.ws.decay[u * DK + tid] = __expf(gval<PERKEY, DK, C>(sm.u.a.gs, C - 1, tid));

    // ------------------------------------------------------- P1b: A and M tiles
    // Wave w computes the tiles of its own row block (i block w, j blocks <= w): the key and
    // query rows of block w are its own registers (B operands), only the j-block keys come
    // from LDS. A is held in registers until the key/gate buffers are dead (barrier #2) and
    // then written over them.
    float atile[NB][4];
    {
        T* mmat = reinterpret_cast<T*>(a.ws.mmat) + u * C * CP;
        if (own) {
            const int ib = w, ref = ib * 16, irow = row;
            // Per-key gate ([LA-Infra] 附1, parts 2-3): the reference point n = ref splits
            // e^{G_i - G_j} = e^{G_i - G_n} e^{G_n - G_j}. For an off-diagonal block (j < n
            // <= i) both exponents are <= 0, so a factor that underflows means a true product
            // below the fp32 range. In the diagonal block (n <= j) the key-side exponent
            // G_n - G_j is >= 0, bounded by the block's own cumulative decay; the split is
            // kept only while that span stays within DIAG_SPAN (both factors then lie well
            // inside the normal fp32 / bf16 range, so the split is exact to rounding).
            // Otherwise the wave computes the diagonal block directly, entry by entry, with
            // the mask applied before the exponential (e^{G_i - G_j} <= 1 for every kept
            // entry), as the page's 对角子块 computation does.
            f32x4 dK = zero4(), dQ = zero4();
            bool direct = false;
            if constexpr (PERKEY) {
                constexpr float DIAG_SPAN = 60.f;
                const int last = min(ref + 15, C - 1);
                bool wide = false;
                for (int ch = lane; ch < DK; ch += WAVE)  // g <= 0: the span is G_n - G_last
                    wide |= !(sm.u.a.gs[ref][ch] - sm.u.a.gs[last][ch] <= DIAG_SPAN);
                direct = __ballot(wide) != 0;  // uniform across the wave
                if (direct) {
                    // lane (g4, r16): row i = irow, its channels kb KB + g4 KPL + e; for each
                    // column j of the block, the partial sums over those channels are
                    // completed across the four lane groups, and the lane whose accumulator
                    // slot holds (j, i) (g4 = (j - ref) / 4) keeps them
#pragma unroll 1
                    for (int jj = 0; jj < 16; jj++) {
                        const int j = ref + jj;
                        float sk = 0.f, sq = 0.f;
#pragma unroll
                        for (int kb = 0; kb < NK; kb++) {
                            const frag kj =
                                MM::load(&sm.u.a.ks[((ib * NK + kb) * 64 + jj + 16 * g4) * KPL]);
#pragma unroll
                            for (int e = 0; e < KPL; e++) {
                                const int ch = kb * KB + g4 * KPL + e;
                                if (ch >= DK) continue;  // zero padding channels
                                float xk, xq, xj;
                                if constexpr (KPL == 1) {
                                    xk = to_f32(kf[kb]); xq = to_f32(qf[kb]); xj = to_f32(kj);
                                } else {
                                    xk = to_f32(kf[kb][e]); xq = to_f32(qf[kb][e]); xj = to_f32(kj[e]);
                                }
                                // masked before the exponential: j > i contributes nothing
                                const float t = j <= irow
                                    ? xj * __expf(sm.u.a.gs[irow][ch] - sm.u.a.gs[j][ch]) : 0.f;
                                sk = fmaf(xk, t, sk);
                                sq = fmaf(xq, t, sq);
                            }
                        }
                        sk += __shfl_xor(sk, 16, WAVE);
                        sk += __shfl_xor(sk, 32, WAVE);
                        sq += __shfl_xor(sq, 16, WAVE);
                        sq += __shfl_xor(sq, 32, WAVE);
#pragma unroll
                        for (int e = 0; e < 4; e++)
                            if (jj == 4 * g4 + e) {
                                dK[e] = sk;
                                dQ[e] = sq;
                            }
                    }
                }
                // the row-side operands k_i e^{G_i - G_n}, q_i e^{G_i - G_n} do not depend on
                // the column block: formed once, in place (the raw rows are dead from here on)
#pragma unroll
                for (int kb = 0; kb < NK; kb++) {
#pragma unroll
                    for (int e = 0; e < KPL; e++) {
                        const int ch = kb * KB + g4 * KPL + e;
                        const float fi =
                            ch < DK ? __expf(sm.u.a.gs[irow][ch] - sm.u.a.gs[ref][ch]) : 0.f;
                        if constexpr (KPL == 1) {
                            kf[kb] = from_f32<T>(to_f32(kf[kb]) * fi);
                            qf[kb] = from_f32<T>(to_f32(qf[kb]) * fi);
                        } else {
                            kf[kb][e] = from_f32<T>(to_f32(kf[kb][e]) * fi);
                            qf[kb][e] = from_f32<T>(to_f32(qf[kb][e]) * fi);
                        }
                    }
                }
            }
#pragma unroll
            for (int jb = 0; jb < NB; jb++) {
                if (jb > ib) continue;
                f32x4 accK = zero4(), accQ = zero4();
                const int jrow = jb * 16 + r16;
                if (PERKEY && direct && jb == ib) {
                    accK = dK;
                    accQ = dQ;
                } else {
#pragma unroll
                    for (int kb = 0; kb < NK; kb++) {
                        const frag ka = MM::load(&sm.u.a.ks[((jb * NK + kb) * 64 + lane) * KPL]);
                        frag fa;
                        if constexpr (PERKEY) {
#pragma unroll
                            for (int e = 0; e < KPL; e++) {
                                const int ch = kb * KB + g4 * KPL + e;
                                float aj = 0.f;
                                if (ch < DK) {  // padded channels contribute zero
                                    const float fj =
                                        __expf(sm.u.a.gs[ref][ch] - sm.u.a.gs[jrow][ch]);
                                    if constexpr (KPL == 1) aj = to_f32(ka) * fj;
                                    else aj = to_f32(ka[e]) * fj;
                                }
                                if constexpr (KPL == 1) fa = from_f32<T>(aj);
                                else fa[e] = from_f32<T>(aj);
                            }
                        } else {
                            fa = ka;
                        }
                        accK = MM::mma(fa, kf[kb], accK);
                        accQ = MM::mma(fa, qf[kb], accQ);
                    }
                }
                // lane holds D[j = jb*16 + 4*g4 + e][i = ib*16 + r16]
                const int i = irow;
                const float gi = PERKEY ? 0.f : sm.u.a.gs[0][i];
                float mrow[4];
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int j = jb * 16 + g4 * 4 + e;
                    float dec = 1.f;
                    if constexpr (!PERKEY) dec = (j <= i) ? __expf(gi - sm.u.a.gs[0][j]) : 0.f;
                    atile[jb][e] = sm.bs[i] * accK[e] * dec;
                    mrow[e] = (j <= i) ? a.scale * accQ[e] * dec : 0.f;
                }
                Frag<T>::template store_run<4>(mmat, i, jb * 16 + g4 * 4, CP, mrow);
            }
        }
        // zero the upper tiles and the padding columns of M, where the scan reads them: it
        // skips the fragments (KB columns) that start right of a row's token block
        for (int idx = tid; idx < C * (CP / 4); idx += PF_THREADS) {
            const int i = idx / (CP / 4), j0 = (idx % (CP / 4)) * 4;
            if ((j0 / 16 > i / 16 || j0 >= C) && (j0 / KB) * KB < 16 * (i / 16 + 1)) {
                float z[4] = {0.f, 0.f, 0.f, 0.f};
                Frag<T>::template store_run<4>(mmat, i, j0, CP, z);
            }
        }
    }
    if constexpr (CONV && PERKEY) {  // wave 0 has the fewest A/M tiles: its V conv here
        if (w == 0 && own) {
#pragma unroll
            for (int f = 2 * NK; f < 2 * NK + NV; f++) conv_frag(f);
            store_vrows();
        }
    }
    lds_barrier();  // #2: keys and gates are dead from here on
    if (own) {
#pragma unroll
        for (int jb = 0; jb < NB; jb++) {
            if (jb > w) continue;
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int j = jb * 16 + g4 * 4 + e;
                if (j < row) sm.u.b.ar[row][j] = atile[jb][e];
            }
        }
    }
    lds_barrier();  // #2b: A in place

    // ------------------------------------------- P2: leaf inverses, V^T, R zero padding
    if (w == 0) {
        // lane (blk, col): column col of (I + A_bb)^{-1} by forward substitution, with the
        // block's strictly lower entries held in registers
        const int blk = g4, col = r16;
        if (blk < NB) {
            const int b0 = blk * 16;
            float av[16][16];
#pragma unroll
            for (int r = 1; r < 16; r++)
#pragma unroll
                for (int kk = 0; kk < r; kk++) av[r][kk] = sm.u.b.ar[b0 + r][b0 + kk];
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; r++) x[r] = (r == col) ? 1.f : 0.f;
#pragma unroll
            for (int r = 1; r < 16; r++) {
                float acc = 0.f;
#pragma unroll
                for (int kk = 0; kk < r; kk++) acc += av[r][kk] * x[kk];
                x[r] -= acc;
            }
#pragma unroll
            for (int r = 0; r < 16; r++) {
                sm.u.b.ar[b0 + r][b0 + col] = x[r];
                sm.u.b.rs[b0 + r][b0 + col] = from_f32<T>(x[r]);
            }
        }
    }
    if constexpr (CONV && PERKEY) {  // the other waves' V conv while wave 0 inverts leaves
        if (w != 0 && own) {
#pragma unroll
            for (int f = 2 * NK; f < 2 * NK + NV; f++) conv_frag(f);
            store_vrows();
        }
    }
    // V^T (when the prep forms U): lane (g4, n) gets V[16w + 4 g4 + e][16 vb + n] (exact in
    // the element type), plus zero padding tokens; per-key gate here, scalar gate after the
    // merges (over A/R)
    auto store_vt = [&]() {
        if (own) {
            const int t0 = w * 16 + g4 * 4;
#pragma unroll
            for (int vb = 0; vb < DV / 16; vb++) {
                const f32x4 vt4 = Ident<T>::template transpose<NV>(vf, vb, idf);
                float vv[4] = {vt4[0], vt4[1], vt4[2], vt4[3]};
                store4<T>(&vt[vb * 16 + r16][t0], vv);
            }
        }
        if constexpr (CP > C) {
            for (int idx = tid; idx < DV * ((CP - C) / 4); idx += PF_THREADS) {
                const int ch = idx / ((CP - C) / 4), t0 = C + (idx % ((CP - C) / 4)) * 4;
                float z[4] = {0.f, 0.f, 0.f, 0.f};
                store4<T>(&vt[ch][t0], z);
            }
        }
    };
    if (PERKEY && uws) store_vt();
    // zeros: R above the diagonal blocks and in the padding columns
    for (int idx = tid; idx < C * (CP / 4); idx += PF_THREADS) {
        const int i = idx / (CP / 4), j0 = (idx % (CP / 4)) * 4;
        if (j0 / 16 > i / 16 || j0 >= C) {
            float z[4] = {0.f, 0.f, 0.f, 0.f};
            store4<T>(&sm.u.b.rs[i][j0], z);
        }
    }
    lds_barrier();  // #3: diagonal blocks of R

    // ------------------------------------------------ P3: 2x2 block merges, fp32 MFMA
    // (L^{-1})_{21} = -L_22^{-1} L_21 L_11^{-1}; the contraction index of each 16x16x4 step
    // is taken as k = 4 g + s so that an accumulator is directly the next B operand.
    if constexpr (NB >= 2) {
        if (w % 2 == 0 && w / 2 < NB / 2) {
            const int lo = (w / 2) * 32, hi = lo + 16;
            f32x4 t1 = zero4();
#pragma unroll
            for (int s4 = 0; s4 < 4; s4++) {
                const int k = 4 * g4 + s4;
                t1 = Mma<float>::mma(sm.u.b.ar[hi + r16][lo + k], sm.u.b.ar[lo + k][lo + r16], t1);
            }
            f32x4 rr = zero4();
#pragma unroll
            for (int s4 = 0; s4 < 4; s4++) {
                const int k = 4 * g4 + s4;
                rr = Mma<float>::mma(sm.u.b.ar[hi + r16][hi + k], t1[s4], rr);
            }
#pragma unroll
            for (int e = 0; e < 4; e++) {
                sm.u.b.ar[hi + 4 * g4 + e][lo + r16] = -rr[e];
                sm.u.b.rs[hi + 4 * g4 + e][lo + r16] = from_f32<T>(-rr[e]);
            }
        }
        lds_barrier();  // #4
    }
    if constexpr (NB >= 4) {
        const int tr = w >> 1, tc = w & 1;
        // T2 = A[32:64, 0:32] R[0:32, 0:32], tile (tr, tc), kept in the strictly upper
        // quarter ar[0:32, 32:64]
        f32x4 t2 = zero4();
#pragma unroll
        for (int kb = 0; kb < 8; kb++) {
            const int k = 4 * kb + g4;
            // R[k][col] is zero above the diagonal blocks (that part of ar was never written)
            const float rb = (tc == 1 && k < 16) ? 0.f : sm.u.b.ar[k][16 * tc + r16];
            t2 = Mma<float>::mma(sm.u.b.ar[32 + 16 * tr + r16][k], rb, t2);
        }
#pragma unroll
        for (int e = 0; e < 4; e++) sm.u.b.ar[16 * tr + 4 * g4 + e][32 + 16 * tc + r16] = t2[e];
        lds_barrier();  // #5
        f32x4 rr = zero4();
#pragma unroll
        for (int kb = 0; kb < 8; kb++) {
            const int k = 4 * kb + g4;
            const float ra = (tr == 0 && k >= 16) ? 0.f : sm.u.b.ar[32 + 16 * tr + r16][32 + k];
            rr = Mma<float>::mma(ra, sm.u.b.ar[k][32 + 16 * tc + r16], rr);
        }
        // the A quarter ar[32:64, 0:32] was last read before barrier #5: overwrite with R_21
#pragma unroll
        for (int e = 0; e < 4; e++) {
            sm.u.b.ar[32 + 16 * tr + 4 * g4 + e][16 * tc + r16] = -rr[e];
            sm.u.b.rs[32 + 16 * tr + 4 * g4 + e][16 * tc + r16] = from_f32<T>(-rr[e]);
        }
    }
    lds_barrier();  // #6: R complete
    if (!PERKEY && uws) {  // uniform across the grid
        store_vt();     // A/R is dead: V^T goes over it
        lds_barrier();  // #7
    }

    // ---------------------------------- P4: -W on MFMA, and U or the scan's operands for it
    // U = R diag(beta) V = diag(beta) V + (R - I) diag(beta) V. R has a unit diagonal, so
    // beta_i V_i is U's leading term: it enters the accumulator in fp32 from the exact V, and
    // only the small off-diagonal part goes through rounded MFMA operands (rounding
    // diag(beta) V itself was the largest single error source of the outputs in the element
    // type). Either the prep forms U here (fp32, in the scan's accumulator order), or the
    // scan forms it the same way from v as it reads it: the prep then stores
    // (R - I) diag(beta) as the A operand of that product (only the fragments at or left of
    // each row's diagonal block; the others are zero and never read) and beta.
    {
        const int kq = g4 * KPL;
        if (own && !uws) {
            T* rr = reinterpret_cast<T*>(a.ws.rr) + u * C * CP;
            const int mb = w, irow = row;
#pragma unroll
            for (int kb = 0; kb < CP / KB; kb++) {
                if (kb * KB >= 16 * (mb + 1)) continue;
                const auto fr = MM::load(&sm.u.b.rs[irow][kb * KB + kq]);
                frag ra;
#pragma unroll
                for (int e = 0; e < KPL; e++) {
                    const int j = kb * KB + kq + e;
                    float x;
                    if constexpr (KPL == 1) x = to_f32(fr);
                    else x = to_f32(fr[e]);
                    x = (j == irow || j >= C) ? 0.f : x * sm.bs[j];
                    if constexpr (KPL == 1) ra = from_f32<T>(x);
                    else ra[e] = from_f32<T>(x);
                }
                *reinterpret_cast<frag*>(rr + ((mb * (CP / KB) + kb) * 64 + lane) * KPL) = ra;
            }
        }
        T* wneg = reinterpret_cast<T*>(a.ws.wneg) + u * C * DKP;
        if constexpr (DKP > DK) {
            for (int idx = tid; idx < C * ((DKP - DK) / 4); idx += PF_THREADS) {
                const int i = idx / ((DKP - DK) / 4), c0 = DK + (idx % ((DKP - DK) / 4)) * 4;
                float z[4] = {0.f, 0.f, 0.f, 0.f};
                Frag<T>::template store_run<4>(wneg, i, c0, DKP, z);
            }
        }
        constexpr int NW = (DK / 16) * NB;  // W^T tiles: (channel block, token block)
        for (int t = w; t < NW; t += PF_WAVES) {
            f32x4 acc = zero4();
            const int nb = t % NB, mb = t / NB;  // nb: token block, mb: channel block
#pragma unroll
            for (int kb = 0; kb < CP / KB; kb++) {
                auto fa = MM::load(&sm.kint[mb * 16 + r16][kb * KB + kq]);
                auto fb = MM::load(&sm.u.b.rs[nb * 16 + r16][kb * KB + kq]);
                acc = MM::mma(fa, fb, acc);
            }
            // lane: W^T[ch = mb*16 + 4*g4 + e][i = nb*16 + r16]
            float nw[4];
#pragma unroll
            for (int e = 0; e < 4; e++) nw[e] = -acc[e];
            Frag<T>::template store_run<4>(wneg, nb * 16 + r16, mb * 16 + g4 * 4, DKP, nw);
        }
        if (uws) {
            float* ut = reinterpret_cast<float*>(a.ws.ut) + u * DV * C;
            constexpr int NU = NB * (DV / 16);  // U tiles: (token block, value block)
            // tile order keeps the R fragments of one token block on one wave; the tiles'
            // A operand (R - I) diag(beta) of that token block is formed once and reused
            frag ua[CP / KB];
            int ua_mb = -1;
            for (int t = w; t < NU; t += PF_WAVES) {
                const int mb = t % NB, nb = t / NB;  // mb: token block, nb: value block
                f32x4 acc;
                {
                    float v4[4];
                    load4<T>(&vt[nb * 16 + r16][mb * 16 + 4 * g4], v4);
                    const f32x4 b4 = *reinterpret_cast<const f32x4*>(&sm.bs[mb * 16 + 4 * g4]);
#pragma unroll
                    for (int e = 0; e < 4; e++) acc[e] = b4[e] * v4[e];
                }
                if (mb != ua_mb) {  // uniform across the wave
                    ua_mb = mb;
                    const int irow = mb * 16 + r16;
#pragma unroll
                    for (int kb = 0; kb < CP / KB; kb++) {
                        const auto fr = MM::load(&sm.u.b.rs[irow][kb * KB + kq]);
#pragma unroll
                        for (int e = 0; e < KPL; e++) {
                            const int j = kb * KB + kq + e;
                            float x;
                            if constexpr (KPL == 1) x = to_f32(fr);
                            else x = to_f32(fr[e]);
                            x = (j == irow || j >= C) ? 0.f : x * sm.bs[j];
                            if constexpr (KPL == 1) ua[kb] = from_f32<T>(x);
                            else ua[kb][e] = from_f32<T>(x);
                        }
                    }
                }
#pragma unroll
                for (int kb = 0; kb < CP / KB; kb++) {
                    if (kb * KB >= 16 * (mb + 1)) continue;  // (R - I) is zero there
                    acc = MM::mma(ua[kb], MM::load(&vt[nb * 16 + r16][kb * KB + kq]), acc);
                }
                // lane: U[i = mb*16 + 4*g4 + e][v = nb*16 + r16], scan accumulator order
                float uu[4] = {acc[0], acc[1], acc[2], acc[3]};
                store4<float>(ut + ((size_t)(nb * NB + mb) * 64 + lane) * 4, uu);
            }
        }
    }
}

// =====================================================================================
// scan kernel: the sequential state pass over chunks
// =====================================================================================
// One workgroup per (sequence, head, value tile) with 2 NB waves (NB = C / 16 token
// blocks); each wave keeps one role for the whole sequence:
//   E wave w < NB      E rows of token block w:  E = U + (-W) S, and the state row blocks
//                      rb = w + j NB of the fp32 state slice, kept in its MFMA accumulators:
//                      S <- Diag(e^{G_C}) S + K_g^T E; then U of its token block for the
//                      next chunk, U = diag(beta) V + ((R - I) diag(beta)) V, from V^T in LDS
//   O wave w >= NB     O rows of token block w - NB: O = Q_in S + M E, and the output
//                      stores; V^T of its token block of the next chunk into LDS
// Per chunk: barrier (S^T in LDS) -> E, Q_in S, next chunk's V^T -> barrier (E in LDS) ->
// state update, S^T back to LDS and the next chunk's U (E waves) while the O waves finish
// M E and store O. Each wave prefetches only its own operands of the next chunk into
// registers (-W, K_g^T rows and (R - I) diag(beta), or Q_in, M and v rows): a single wave
// pulls only a small share of a CU's vector-memory bandwidth, so the per-chunk operand
// stream is spread over all waves of the workgroup. U never leaves the CU: forming it here
// instead of in the prep saves the prep's read of v and the U round trip through HBM
// (fp32, 4 bytes per value, against v's 2 for bf16). The E waves form it after issuing
// their S^T stores, so its products run while those complete; in the output waves, whose
// chunk step is the longer one, the same work lengthened every chunk.
template <int C>
struct ScanShape {
    static constexpr int NB = C / 16;
    static constexpr int NWV = 2 * NB;
    static constexpr int THREADS = NWV * WAVE;
};

template <typename T, int DK, int DV, int C, bool PERKEY, bool EROLE, int NVB>
struct ScanOps {
    using F = PfCfg<T, DK, DV, C>;
    using frag = typename F::MM::frag;
    static constexpr int NK = F::DKP / F::KB;    // k-steps over (padded) d_k
    static constexpr int NK2 = F::CP / F::KB;    // k-steps over the chunk
    static constexpr int NB = C / 16;
    static constexpr int RB = DK / 16;
    static constexpr int RBW = (RB + NB - 1) / NB;   // state row blocks per E wave
    // with RB a multiple of the E-wave count every E wave owns full row blocks and the loop
    // stays branch-free (the compiler then waits only for the operands it needs)
    static constexpr bool RB_FULL = RB % NB == 0;
    static constexpr int NVF = (SCAN_BV * NVB + F::KB - 1) / F::KB;  // v row fragments
    frag a[NK];                    // -W rows (E wave) or Q_in rows (O wave)
    frag am[EROLE ? 1 : NK2];      // M rows (O wave)
    frag ak[EROLE ? RBW : 1][NK2]; // K_g^T rows of the wave's state row blocks (E wave)
    f32x4 dec[PERKEY ? RBW : 1];   // per key: e^{G_C} of the lane's 4 state rows
    float dec0;                    // scalar gate: e^{G_C}
    // E wave: with 16-column tiles U of the token block, formed by the prep; with wider
    // ones the next chunk's (R - I) diag(beta) rows and beta of the lane's 4 accumulator rows
    f32x4 u;
    frag ar[EROLE ? NK2 : 1];
    f32x4 bt;
    f32x4 qs;  // O wave reading q itself: the output row factors of the lane's 4 rows
};

// Every lane issues every load below (a lane without a row reads the first element of the
// source and drops it; fragments right of the diagonal block, which are zero, reload the
// first one, a cache hit), so the number of loads per chunk is fixed: the compiler's wait
// counts then stay exact, where skipped loads made it wait for the next chunk's prefetches
// as well.
// The next chunk's U operands of token block mb for an E wave: (R - I) diag(beta) rows and
// beta.
template <typename T, int DK, int DV, int C, bool PERKEY, int NVB>
__device__ __forceinline__ void scan_load_u_in(ScanOps<T, DK, DV, C, PERKEY, true, NVB>& op,
                                               const PrefillArgs& a, size_t un, int mb) {
    using O = ScanOps<T, DK, DV, C, PERKEY, true, NVB>;
    using F = PfCfg<T, DK, DV, C>;
    using MM = typename F::MM;
    const int lane = lane_id(), g = lane >> 4;
    const T* rr = reinterpret_cast<const T*>(a.ws.rr) + un * C * F::CP;
#pragma unroll
    for (int kt = 0; kt < O::NK2; kt++)
        op.ar[kt] = MM::load(Frag<T>::ptr(rr, mb, kt * F::KB < 16 * (mb + 1) ? kt : 0, F::CP, lane));
    op.bt = *reinterpret_cast<const f32x4*>(a.ws.beta + un * C + mb * 16 + 4 * g);
}
// v rows of an O wave's token block as row fragments over the tile's columns; vrow is the
// lane's row at the tile's first column, or null for a row past the sequence end.
template <typename T, int NVF, int BV>
__device__ __forceinline__ void scan_load_v(typename Mma<T>::frag (&vr)[NVF], const T* vrow,
                                            const T* vsafe) {
    using MM = Mma<T>;
    const int g = lane_id() >> 4;
#pragma unroll
    for (int f = 0; f < NVF; f++) {
        const int col = f * MM::KB + g * MM::KPL;
        const bool ok = vrow != nullptr && col < BV;
        const auto x = MM::load(ok ? vrow + col : vsafe);
        vr[f] = ok ? x : MM::zero();
    }
}

// Operand loads of one chunk for one wave, in two parts issued at different points of the
// previous chunk: part 0 (first needed: -W and U, or Q_in) and part 1 (K_g^T rows and decay,
// or M). Issuing a wave's whole set at once stalls it on a full vector-memory queue.
// QRAW: the O waves read q rows (qrow: the lane's row, or null past the sequence end) and
// the row factors instead of Q_in. UW: the E waves read U (fp32, formed by the prep) for
// the tile at vcol0, else the operands that form it here.
template <int PART, bool QRAW, bool UW, typename T, int DK, int DV, int C, bool PERKEY, bool EROLE, int NVB>
__device__ __forceinline__ void scan_load_ops(ScanOps<T, DK, DV, C, PERKEY, EROLE, NVB>& op,
                                              const PrefillArgs& a, size_t u, size_t un,
                                              int vcol0, const T* qrow, int mb, int w) {
    using O = ScanOps<T, DK, DV, C, PERKEY, EROLE, NVB>;
    using F = PfCfg<T, DK, DV, C>;
    using MM = typename F::MM;
    constexpr int CP = F::CP;
    const int lane = lane_id();
    const float* dec = a.ws.decay + u * DK;
    if constexpr (PART == 0) {
        if constexpr (EROLE) {
            const T* wneg = reinterpret_cast<const T*>(a.ws.wneg) + u * C * F::DKP;
#pragma unroll
            for (int kb = 0; kb < O::NK; kb++) op.a[kb] = MM::load(Frag<T>::ptr(wneg, mb, kb, F::DKP, lane));
            if constexpr (UW) {  // U of this lane's accumulator slots (fp32)
                const float* ut = reinterpret_cast<const float*>(a.ws.ut) + u * DV * C;
                op.u = *reinterpret_cast<const f32x4*>(ut + ((size_t)((vcol0 / 16) * F::NB + mb) * 64 + lane) * 4);
            }
        } else if constexpr (QRAW) {  // q rows as they are, padded channels zero
            const T* qsafe = reinterpret_cast<const T*>(a.q);
#pragma unroll
            for (int kb = 0; kb < O::NK; kb++) {
                const int col = kb * F::KB + (lane >> 4) * F::KPL;
                const bool ok = qrow != nullptr && col < DK;
                const auto x = MM::load(ok ? qrow + col : qsafe);
                op.a[kb] = ok ? x : MM::zero();
            }
            op.qs = *reinterpret_cast<const f32x4*>(a.ws.qs + u * C + mb * 16 + (lane >> 4) * 4);
        } else {
            const T* qin = reinterpret_cast<const T*>(a.ws.qin) + u * C * F::DKP;
#pragma unroll
            for (int kb = 0; kb < O::NK; kb++) op.a[kb] = MM::load(Frag<T>::ptr(qin, mb, kb, F::DKP, lane));
        }
    } else {
        if constexpr (EROLE) {
            if constexpr (!PERKEY) op.dec0 = dec[0];
            const T* kgt = reinterpret_cast<const T*>(a.ws.kgt) + u * DK * CP;
#pragma unroll
            for (int j = 0; j < O::RBW; j++) {
                const int rb = w + j * O::NB;
                if (O::RB_FULL || rb < O::RB) {
#pragma unroll
                    for (int kt = 0; kt < O::NK2; kt++)
                        op.ak[j][kt] = MM::load(Frag<T>::ptr(kgt, rb, kt, CP, lane));
                    if constexpr (PERKEY)  // 4 distinct 16-byte words per wave: one cache line
                        op.dec[j] = *reinterpret_cast<const f32x4*>(dec + rb * 16 + (lane >> 4) * 4);
                }
            }
            if constexpr (!UW) scan_load_u_in(op, a, un, mb);
        } else {
            const T* mm = reinterpret_cast<const T*>(a.ws.mmat) + u * C * CP;
            // M is lower triangular: the fragments starting right of token block mb would
            // hold only zeros; the prep leaves them unwritten and they are never multiplied
            // here (mb is uniform across the wave). In their place the wave reloads its first
            // fragment, to keep the number of loads fixed (see scan_load_u_in).
#pragma unroll
            for (int kt = 0; kt < O::NK2; kt++)
                op.am[kt] = MM::load(Frag<T>::ptr(mm, mb, kt * F::KB < 16 * (mb + 1) ? kt : 0, CP, lane));
        }
    }
}

// NVB value tiles of 16 columns per workgroup: 1 gives the most workgroups (a single long
// sequence), 2-8 divide the per-column operand stream when there are many (sequence, head)
// units to fill the chip with.
// CKPT: also export the states a checkpoint list asks for (its own instantiation, so the
// pass without checkpoints carries none of the bookkeeping).
// QRAW: the output waves multiply q itself by S and scale each row by the prep's factor
// s e^{G_i} / |q_i| (scalar gate, q given, tiles wider than 16 columns; PrefillArgs::q_raw).
// SEG (segmented scan, PrefillArgs::seg = K; a sequence of n chunks is cut into
// k = seg_count(n, K) segments at seg_bound): 0 = the whole sequence; 1 = its first segment,
// from the initial state, ending with the state at the first boundary in the workspace (or,
// for a sequence left in one piece, the final state in the pool as usual); 2 = its later
// segment sidx (1 <= sidx < k), with NVB = 2: the 16-column value tile run from a zero state
// (outputs O0, fp32 in the workspace, and final state Delta) beside the matching 16 columns
// of the identity run (state I, U = 0: outputs L and final state P, the segment's
// transition). Every quantity of the pass is affine in the incoming state, so with S_j the
// state at the start of segment j the true outputs are O0 + L S_j and the state at its end
// is P S_j + Delta, which the chain and combine passes form.
// (unit, vtile): the workgroup's (sequence, head) and value tile, as its kernel maps them.
template <typename T, int DK, int DV, int C, bool PERKEY, int NVB, bool CKPT, bool QRAW, int SEG>
__device__ __forceinline__ void prefill_scan_body(const PrefillArgs& a, const int unit,
                                                  const int vtile, const int sidx) {
    using F = PfCfg<T, DK, DV, C>;
    using MM = typename F::MM;
    using frag = typename MM::frag;
    constexpr int KB = F::KB, KPL = F::KPL, CP = F::CP, NB = F::NB;
    constexpr int THREADS = ScanShape<C>::THREADS;
    constexpr int RB = DK / 16, RBW = (RB + NB - 1) / NB;   // state row blocks per E wave
    constexpr bool RB_FULL = RB % NB == 0;
    constexpr int BV = SCAN_BV * NVB;
    constexpr bool HYB = SEG == 2;  // value tile + identity tile
    static_assert(!HYB || NVB == 2, "the second segment pairs two tiles");
    static_assert(SEG == 0 || (!CKPT && !QRAW), "segmented scan: no checkpoints, Q_in");
    constexpr int TW = HYB ? SCAN_BV : BV;  // value columns of the workgroup
    __shared__ __align__(16) T st[BV][F::LDK];   // S^T slice (MFMA B operand)
    __shared__ __align__(16) T et[BV][F::LDC];   // E^T slice
    __shared__ __align__(16) T ot[NB][NVB][16][16];  // O tiles of the O waves, row-major
    constexpr bool UWS = NVB == 1 || HYB;  // U from the workspace (formed by the prep)
    __shared__ __align__(16) T vt[UWS ? 1 : BV][F::LDC];  // V^T slice of the next chunk

    const int H = a.H;
    if (unit >= a.n_seqs * H) return;
    const int n = unit / H, h = unit - (unit / H) * H;
    // the wave index is uniform across a wave; saying so keeps role and checkpoint branches
    // scalar
    const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(wave_id());
    const int r16 = lane & 15, g = lane >> 4;
    const int kq = g * KPL;
    const int vcol0 = vtile * TW;
    // clamps keep inconsistent cu_seqlens inside the workspace and the token range
    int c_first, c_last1;
    if (a.n_seqs <= SEQ_INLINE_MAX) {
        const WaveSeqTable t = wave_seq_table(a.cu_seqlens, a.n_seqs, C);
        c_first = __builtin_amdgcn_readlane(t.excl, n);
        c_last1 = __builtin_amdgcn_readlane(t.incl, n);
    } else {
        c_first = a.ws.seq_first[n];
        c_last1 = a.ws.seq_first[n + 1];
    }
    // this workgroup's chunks [c_begin, c_end); token offsets count from c_first
    const int c_seq_end = (int)min((int64_t)c_last1, a.ws.max_chunks);
    const int kseg = SEG != 0 ? seg_count(c_seq_end - c_first, a.seg) : 1;
    if (HYB && sidx >= kseg) return;  // no such segment (uniform across the workgroup)
    const int c_begin = SEG == 2 ? seg_bound(c_first, c_seq_end, sidx, kseg) : c_first;
    const int c_end = SEG == 0 ? c_seq_end : seg_bound(c_first, c_seq_end, sidx + 1, kseg);
    const bool split = SEG == 1 && kseg > 1;  // first segment of a split sequence
    const int t_begin = a.cu_seqlens[n], t_end = min(a.cu_seqlens[n + 1], a.total_tokens);
    const int slot = a.slots[n];
    const bool valid = slot >= 0 && slot < a.n_slots;
    const bool init = !HYB && valid && a.has_init != nullptr && a.has_init[n] != 0;
    float* S = valid ? a.state_pool + ((size_t)slot * H + h) * DK * DV : nullptr;

    // state slice in the E waves' accumulators:
    //   acc_s[j][v][e] = S[16 rb + 4 g + e][vcol0 + 16 v + r16],  rb = w + j NB  (w < NB)
    const bool ewave = w < NB;
    f32x4 acc_s[RBW][NVB];
#pragma unroll
    for (int j = 0; j < RBW; j++) {
        const int rb = w + j * NB;
#pragma unroll
        for (int v = 0; v < NVB; v++) {
            acc_s[j][v] = zero4();
            if (ewave && rb < RB) {
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int row = rb * 16 + 4 * g + e;
                    if (HYB)  // value tile from zero, identity tile from columns of I
                        acc_s[j][v][e] = v == 1 && row == vcol0 + r16 ? 1.f : 0.f;
                    else
                        acc_s[j][v][e] = init ? S[(size_t)row * DV + vcol0 + 16 * v + r16] : 0.f;
                    st[16 * v + r16][row] = from_f32<T>(acc_s[j][v][e]);
                }
            }
        }
    }
    if constexpr (CP > C) {  // token padding of E^T and V^T stays zero
        for (int idx = threadIdx.x; idx < BV * (CP - C); idx += THREADS) {
            et[idx / (CP - C)][C + idx % (CP - C)] = from_f32<T>(0.f);
            if constexpr (!UWS) vt[idx / (CP - C)][C + idx % (CP - C)] = from_f32<T>(0.f);
        }
    }
    if constexpr (F::DKP > DK) {  // padded state rows stay zero
        for (int idx = threadIdx.x; idx < BV * (F::DKP - DK); idx += THREADS)
            st[idx / (F::DKP - DK)][DK + idx % (F::DKP - DK)] = from_f32<T>(0.f);
    }

    T* out = reinterpret_cast<T*>(a.o);
    T* dump = reinterpret_cast<T*>(a.ws.dump) + 4 * lane;  // 64 lanes x 4 elements <= 1 KiB

    // Output stores (o, exported and final states). With one 16-column tile per workgroup
    // they carry the non-temporal hint: their write-back then happens during this scan,
    // which leaves HBM mostly idle, instead of during the next kernel (on the 8192-token,
    // 16-head call the next call's prep ran 5-6 µs faster). Wider tiles keep plain stores:
    // without the caches merging the separate 32-byte pieces of a row, their write traffic
    // grew by 38-45 % and the scan slowed.
    constexpr bool NT = NVB == 1;
    // the E waves write their state rows (fp32, from the accumulators) to a pool slot
    auto store_state = [&](float* dst) {
#pragma unroll
        for (int j = 0; j < RBW; j++) {
            const int rb = w + j * NB;
            if (rb < RB) {
#pragma unroll
                for (int v = 0; v < NVB; v++)
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        float* p = &dst[(size_t)(rb * 16 + 4 * g + e) * DV + vcol0 + 16 * v + r16];
                        if constexpr (NT) __builtin_nontemporal_store(acc_s[j][v][e], p);
                        else *p = acc_s[j][v][e];
                    }
            }
        }
    };
    // Checkpoints (E waves). ck.chunk is the chunk whose completion gives the next stored
    // entry (INT_MAX: none). Entries are fetched 64 at a time, one per lane, and read back
    // with readlane, so finding the next one issues no load unless a batch runs out.
    struct {
        int next, end, base, pv, sv, high, chunk, slot;
    } ck{0, 0, 0, 0, -1, INT_MIN, INT_MAX, -1};
    const int len = t_end - t_begin;
    auto ck_fetch = [&]() {  // the batch of entries starting at ck.next
        ck.base = ck.next;
        const int i = ck.base + lane;
        ck.pv = i < ck.end ? a.ckpt_pos[i] : 0;
        ck.sv = i < ck.end ? a.ckpt_slots[i] : -1;
    };
    // Entry i is stored iff its offset p is usable (0 < p <= length, p a multiple of C or
    // the length) and no earlier entry of the sequence has a larger offset.
    auto ck_advance = [&]() {
        ck.chunk = INT_MAX;
        while (ck.next < ck.end) {
            if (ck.next - ck.base == WAVE) ck_fetch();
            const int p = __builtin_amdgcn_readlane(ck.pv, ck.next - ck.base);
            const int sl = __builtin_amdgcn_readlane(ck.sv, ck.next - ck.base);
            ck.next++;
            const bool use = p > 0 && p <= len && (p % C == 0 || p == len) && p >= ck.high;
            ck.high = max(ck.high, p);
            if (use) {
                ck.chunk = c_first + (p + C - 1) / C - 1;
                ck.slot = sl;
                break;
            }
        }
    };
    if (CKPT && ewave) {
        ck.next = max(a.ckpt_cu[n], 0);
        ck.end = min(a.ckpt_cu[n + 1], a.n_ckpt);
        ck_fetch();
        ck_advance();
    }
    auto ck_hit = [&](int c) {  // after the state update of chunk c == ck.chunk
        do {
            if (ck.slot >= 0 && ck.slot < a.n_slots)
                store_state(a.state_pool + ((size_t)ck.slot * H + h) * DK * DV);
            ck_advance();
        } while (ck.chunk == c);
    };

    // U of a chunk in two steps one barrier apart: each O wave writes V^T of its token block
    // (exact in the element type) into vt; then, with all of V^T there, each E wave forms
    // U = diag(beta) V + ((R - I) diag(beta)) V of its token block in registers.
    const T* const vsrc = reinterpret_cast<const T*>(a.conv_width != 0 ? a.ws.vbuf : a.v);
    const int mbo = w - NB;  // an O wave's token block
    // the lane's v row of chunk cc (O waves) at the tile's first column; null past the end
    // the lane's q row of chunk cc (O waves); null past the end
    auto qrow_of = [&](int cc) -> const T* {
        const int tok0 = t_begin + (cc - c_first) * C;
        const int i = mbo * 16 + r16;
        if (i >= min(C, t_end - tok0) || tok0 + i < 0) return nullptr;
        return reinterpret_cast<const T*>(a.q) + ((size_t)(tok0 + i) * H + h) * DK;
    };
    auto vrow_of = [&](int cc) -> const T* {
        const int tok0 = t_begin + (cc - c_first) * C;
        const int i = mbo * 16 + r16;
        if (i >= min(C, t_end - tok0) || tok0 + i < 0) return nullptr;
        if (a.conv_width != 0) return vsrc + ((size_t)(cc * H + h) * C + i) * DV + vcol0;
        return vsrc + ((size_t)(tok0 + i) * H + h) * DV + vcol0;
    };
    frag idf[Ident<T>::N];
    Ident<T>::make(idf);
    using EOps = ScanOps<T, DK, DV, C, PERKEY, true, NVB>;
    constexpr int NVF = EOps::NVF;
    auto load_v = [&](frag (&vr)[NVF], int cc) { scan_load_v<T, NVF, BV>(vr, vrow_of(cc), vsrc); };
    auto stage_vt = [&](const frag (&vr)[NVF]) {
#pragma unroll
        for (int vb = 0; vb < NVB; vb++) {
            const f32x4 t4 = Ident<T>::template transpose<NVF>(vr, vb, idf);
            float vv[4] = {t4[0], t4[1], t4[2], t4[3]};
            store4<T>(&vt[vb * 16 + r16][mbo * 16 + 4 * g], vv);
        }
    };
    f32x4 un[NVB];  // E wave: U of its token block, next chunk
    auto form_u = [&](const EOps& op) {
#pragma unroll
        for (int v = 0; v < NVB; v++) {
            float v4[4];
            load4<T>(&vt[16 * v + r16][w * 16 + 4 * g], v4);
            f32x4 acc;
#pragma unroll
            for (int e = 0; e < 4; e++) acc[e] = op.bt[e] * v4[e];
#pragma unroll
            for (int kt = 0; kt < EOps::NK2; kt++) {
                if (kt * KB >= 16 * (w + 1)) continue;  // (R - I) is zero there
                acc = MM::mma(op.ar[kt], MM::load(&vt[16 * v + r16][kt * KB + kq]), acc);
            }
            un[v] = acc;
        }
    };

    // the sequential pass for one role; both roles meet the same two barriers per chunk
    auto run = [&](auto role) {
        constexpr bool E = decltype(role)::value;
        using O = ScanOps<T, DK, DV, C, PERKEY, E, NVB>;
        const int mb = E ? w : w - NB;
        auto update_state = [&](const O& cur) {  // E waves, after the E barrier
            // one value tile at a time: its E^T fragments are live only for that tile
#pragma unroll
            for (int v = 0; v < NVB; v++) {
                frag fe[O::NK2];
#pragma unroll
                for (int kt = 0; kt < O::NK2; kt++) fe[kt] = MM::load(&et[16 * v + r16][kt * KB + kq]);
#pragma unroll
                for (int j = 0; j < RBW; j++) {
                    const int rb = w + j * NB;
                    if (RB_FULL || rb < RB) {
#pragma unroll
                        for (int e = 0; e < 4; e++)
                            acc_s[j][v][e] *= PERKEY ? cur.dec[PERKEY ? j : 0][e] : cur.dec0;
#pragma unroll
                        for (int kt = 0; kt < O::NK2; kt++)
                            acc_s[j][v] = MM::mma(cur.ak[j][kt], fe[kt], acc_s[j][v]);  // + K_g^T E
                        float sv[4] = {acc_s[j][v][0], acc_s[j][v][1], acc_s[j][v][2], acc_s[j][v][3]};
                        store4<T>(&st[16 * v + r16][rb * 16 + 4 * g], sv);
                    }
                }
            }
        };
        // operands of chunk c + 1 are loaded while chunk c is computed; prefetch indices are
        // clamped to the last chunk so every load is unconditional
        const int clast = c_end - 1;
        auto ld = [&](auto part, O& op, int c) {  // U operands: of the chunk after c
            constexpr int PART = decltype(part)::value;
            const int cc = min(c, clast);
            scan_load_ops<PART, QRAW, UWS, T, DK, DV, C, PERKEY, E, NVB>(
                op, a, (size_t)cc * H + h, (size_t)min(c + 1, clast) * H + h, vcol0,
                QRAW && !E && PART == 0 ? qrow_of(cc) : nullptr, mb, w);
        };
        using part0 = std::integral_constant<int, 0>;
        using part1 = std::integral_constant<int, 1>;
        // O waves: v rows in a ring of two slots by chunk parity; at chunk c slot c holds
        // V_{c+1}, which is staged and replaced by V_{c+3}: two chunks of latency cover the
        // rows' trip from HBM (with one, the waves stalled on them every chunk)
        auto step = [&](const O& cur, O& nxt, frag (&vq)[NVF], int c) {
            lds_barrier();  // st holds S_c^T
            ld(part1(), nxt, c + 1);
            sched_fence();
            f32x4 acc[NVB];
#pragma unroll
            for (int v = 0; v < NVB; v++)
                acc[v] = E ? (UWS ? (HYB && v == 1 ? zero4() : cur.u) : un[v]) : zero4();
#pragma unroll
            for (int kb = 0; kb < O::NK; kb++)
#pragma unroll
                for (int v = 0; v < NVB; v++) {
                    auto fb = MM::load(&st[16 * v + r16][kb * KB + kq]);
                    acc[v] = MM::mma(cur.a[kb], fb, acc[v]);  // E: U - W S;  O: Q_in S
                }
            if constexpr (E) {
#pragma unroll
                for (int v = 0; v < NVB; v++) {
                    float ev[4] = {acc[v][0], acc[v][1], acc[v][2], acc[v][3]};
                    store4<T>(&et[16 * v + r16][mb * 16 + 4 * g], ev);
                }
            } else if constexpr (QRAW) {  // O = diag(s e^{G} / |q|) q S + M E
#pragma unroll
                for (int v = 0; v < NVB; v++)
#pragma unroll
                    for (int e = 0; e < 4; e++) acc[v][e] *= cur.qs[e];
            }
            if constexpr (!E && !UWS) {
                stage_vt(vq);  // V^T of chunk c + 1
                load_v(vq, min(c + 3, clast));
            }
            lds_barrier();  // et holds E_c, vt V_{c+1}^T
            ld(part0(), nxt, c + 1);
            sched_fence();
            if constexpr (!E) {
#pragma unroll
                for (int kt = 0; kt < O::NK2; kt++) {
                    if (kt * KB >= 16 * (mb + 1)) continue;  // zero fragment of M
#pragma unroll
                    for (int v = 0; v < NVB; v++) {
                        auto fb = MM::load(&et[16 * v + r16][kt * KB + kq]);
                        acc[v] = MM::mma(cur.am[kt], fb, acc[v]);  // + M E
                    }
                }
                if constexpr (HYB) {
                    // O0 (fp32) over this chunk's U, in the same accumulator order: the E
                    // waves took U_c into their E rows before the E barrier. L (bf16) as
                    // row-major fragments of a C x d_k A operand, through LDS like O below.
                    const size_t uo = (size_t)c * H + h;
                    float* o0 = reinterpret_cast<float*>(a.ws.ut) + uo * DV * C;
                    *reinterpret_cast<f32x4*>(o0 + ((size_t)((vcol0 / 16) * NB + mb) * 64 + lane) * 4) = acc[0];
#pragma unroll
                    for (int e = 0; e < 4; e++) ot[mb][1][4 * g + e][r16] = from_f32<T>(acc[1][e]);
                    asm volatile("" ::: "memory");  // LDS accesses of one wave complete in order
                    float lv[4];
                    load4<T>(&ot[mb][1][lane >> 2][(lane & 3) * 4], lv);
                    T* lb = reinterpret_cast<T*>(a.ws.lbuf) + uo * C * F::DKP;
                    Frag<T>::template store_run<4>(lb, mb * 16 + (lane >> 2), vcol0 + (lane & 3) * 4, F::DKP, lv);
                    return;
                }
                // the accumulator holds 4 tokens of one column per lane; a row-major pass
                // through LDS lets every lane store 4 adjacent columns of one token at once
                const int tok0 = t_begin + (c - c_first) * C;
                const int len = min(C, t_end - tok0);
#pragma unroll
                for (int v = 0; v < NVB; v++)
#pragma unroll
                    for (int e = 0; e < 4; e++) ot[mb][v][4 * g + e][r16] = from_f32<T>(acc[v][e]);
                asm volatile("" ::: "memory");  // LDS accesses of one wave complete in order
                const int orow = lane >> 2, oc = (lane & 3) * 4;
                const int i = mb * 16 + orow;
#pragma unroll
                for (int v = 0; v < NVB; v++) {
                    float ov[4];
                    load4<T>(&ot[mb][v][orow][oc], ov);
                    // tokens past the sequence end (or, with cu_seqlens that break the
                    // contract, before token 0) go to a scratch area instead of a branch
                    T* dst = i < len && tok0 + i >= 0
                                 ? out + ((size_t)(tok0 + i) * H + h) * DV + vcol0 + 16 * v + oc
                                 : dump;
                    if constexpr (NT) store4_nt<T>(dst, ov);
                    else store4<T>(dst, ov);
                }
            } else {
                update_state(cur);
                if constexpr (!UWS) form_u(cur);  // U_{c+1}, while the S^T stores complete
                if constexpr (CKPT)
                    if (c == ck.chunk) ck_hit(c);
            }
        };
        O op0, op1;
        frag vqa[NVF], vqb[NVF];
        ld(part0(), op0, c_begin);
        ld(part1(), op0, c_begin);
        if constexpr (!E && !UWS) {
            load_v(vqa, min(c_begin + 1, clast));
            load_v(vqb, min(c_begin + 2, clast));
        }
        // two chunks per iteration, then the odd one (a break in the middle of the body
        // compiles to a slower loop)
        int c = c_begin;
        for (; c + 1 < c_end; c += 2) {
            step(op0, op1, vqa, c);
            step(op1, op0, vqb, c + 1);
        }
        if (c < c_end) step(op0, op1, vqa, c);
    };
    if (c_begin < c_end) {
        if constexpr (!UWS) {  // U of the first chunk (the loop forms the later ones ahead)
            if (!ewave) {
                frag v0[NVF];
                load_v(v0, c_begin);
                stage_vt(v0);
                lds_barrier();
            } else {
                EOps op;
                scan_load_u_in(op, a, (size_t)c_begin * H + h, w);
                lds_barrier();
                form_u(op);
            }
        }
        if (w < NB) {
            // an E wave shares its SIMD with an O wave; issuing its instructions first keeps
            // the state chain, which every chunk waits on, ahead of the output work
            __builtin_amdgcn_s_setprio(1);
            run(std::integral_constant<bool, true>());
        } else {
            run(std::integral_constant<bool, false>());
        }
    }
    if (!ewave) return;
    if constexpr (SEG == 2) {  // Delta (value tile) and P (identity tile), columns vcol0..+16
        const size_t bu = (size_t)(sidx - 1) * a.n_seqs * H + unit;  // boundary sidx
        float* dl = a.ws.delta + bu * DK * DV;
        float* pt = a.ws.ptrans + bu * DK * DV;
#pragma unroll
        for (int j = 0; j < RBW; j++) {
            const int rb = w + j * NB;
            if (rb < RB) {
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const size_t idx = (size_t)(rb * 16 + 4 * g + e) * DV + vcol0 + r16;
                    dl[idx] = acc_s[j][0][e];
                    pt[idx] = acc_s[j][1][e];
                }
            }
        }
    } else if (split) {  // the state at the first boundary: fp32, and bf16 transposed
        store_state(a.ws.smid + (size_t)unit * DK * DV);
        T* smt = reinterpret_cast<T*>(a.ws.smidt) + (size_t)unit * DV * DK;
#pragma unroll
        for (int j = 0; j < RBW; j++) {
            const int rb = w + j * NB;
            if (rb < RB) {
                float sv[4] = {acc_s[j][0][0], acc_s[j][0][1], acc_s[j][0][2], acc_s[j][0][3]};
                store4<T>(smt + (size_t)(vcol0 + r16) * DK + rb * 16 + 4 * g, sv);
            }
        }
    } else if (valid) {
        store_state(S);
    }
}

// XCD-aware unit mapping: all value tiles of a (sequence, head) on one XCD, as workgroups
// are dispatched to the 8 XCDs in turn (the grid is a multiple of 8 units).
template <typename T, int DK, int DV, int C, bool PERKEY, int NVB, bool CKPT, bool QRAW>
__global__ __launch_bounds__(ScanShape<C>::THREADS) void prefill_scan_kernel(PrefillArgs a) {
    constexpr int NVT = DV / (SCAN_BV * NVB);
    const int xcd = (int)blockIdx.x & 7, jj = (int)blockIdx.x >> 3;
    prefill_scan_body<T, DK, DV, C, PERKEY, NVB, CKPT, QRAW, 0>(a, (jj / NVT) * 8 + xcd,
                                                                jj % NVT, 0);
}
// All segments in one launch, on the CUs a one-segment scan leaves idle: virtual unit
// vu = s units + unit is segment s of (sequence, head) unit, mapped to XCDs as above (the
// segments of a unit read different chunks, so they need not share an XCD); s = 0 runs first
// segments (one 16-column tile), s >= 1 later ones (value tile + identity tile).
template <typename T, int D, int C, bool PERKEY>
__global__ __launch_bounds__(ScanShape<C>::THREADS) void prefill_scan_seg_kernel(PrefillArgs a) {
    constexpr int NVT = D / SCAN_BV;
    const int units = a.n_seqs * a.H;
    const int xcd = (int)blockIdx.x & 7, jj = (int)blockIdx.x >> 3;
    const int vu = (jj / NVT) * 8 + xcd, vtile = jj % NVT;
    if (vu >= a.seg * units) return;
    const int sidx = vu / units, unit = vu - sidx * units;
    if (sidx == 0)
        prefill_scan_body<T, D, D, C, PERKEY, 1, false, false, 1>(a, unit, vtile, 0);
    else
        prefill_scan_body<T, D, D, C, PERKEY, 2, false, false, 2>(a, unit, vtile, sidx);
}

// =====================================================================================
// chain and combine passes of the segmented scan (bf16)
// =====================================================================================
// Per sequence (lane n of a wave): its chunk range [c0, c1) (clamped as in the scan), its
// segment count k, and the chunks of its later segments, [seg_bound(1), c1), counted (nbl)
// and prefixed over the sequences (pex exclusive, pin inclusive).
struct SegTable {
    int c0, c1, k, nbl, pex, pin;
};
__device__ __forceinline__ SegTable seg_table(const PrefillArgs& a, int C) {
    const WaveSeqTable t = wave_seq_table(a.cu_seqlens, a.n_seqs, C);
    SegTable r;
    r.c0 = t.excl;
    r.c1 = (int)min((int64_t)t.incl, a.ws.max_chunks);
    const bool live = lane_id() < a.n_seqs;
    r.k = live ? seg_count(r.c1 - r.c0, a.seg) : 1;
    r.nbl = live && r.k > 1 ? max(0, r.c1 - seg_bound(r.c0, r.c1, 1, r.k)) : 0;
    r.pin = r.nbl;
#pragma unroll
    for (int off = 1; off < WAVE; off <<= 1) {
        const int y = __shfl_up(r.pin, off, WAVE);
        if (lane_id() >= off) r.pin += y;
    }
    r.pex = r.pin - r.nbl;
    return r;
}

constexpr int CB_THREADS = 256;
// Chain pass (K > 2): the state at the start of each later segment but the last,
// S_{j+1} = P_j S_j + Delta_j for j = 1 .. k - 2, from S_1 (the first segment's end state), on
// fp32 MFMA. One workgroup per (sequence, head, 16 state columns): each column slice of the
// state evolves on its own, kept transposed in LDS across the steps. Each S_{j+1} is written
// in bf16 transposed (the combine's output operand), and S_{k-1} also in fp32, from which
// the combine forms the final state. The steps form a dependent chain, so each one's
// latency counts: its B operands come from LDS as 16-byte reads issued together before the
// products, and the next step's P and Delta (which do not depend on the chain) are loaded
// before this step's products.
template <typename T, int DK, int DV, int C>
__global__ __launch_bounds__(CB_THREADS) void prefill_seg_chain_kernel(PrefillArgs a) {
    using MF = Mma<float>;
    constexpr int NT = DV / 16, NW = CB_THREADS / WAVE, RBW = DK / 16 / NW, NQ = DK / 16;
    constexpr int LDS_T = DK + 4;  // row stride of the transposed slice (floats, 16-byte rows)
    static_assert(DK % (16 * NW) == 0, "state row blocks spread evenly over the waves");
    static_assert((DK * 16 / 4) % CB_THREADS == 0, "S_1 slice in whole 16-byte loads");
    __shared__ __align__(16) float slt[16][LDS_T];  // slt[c][key] = S_j[key][16 tv + c]
    const int H = a.H, nu = a.n_seqs * H;
    // the NT slices of a (sequence, head) on one XCD, as in the scan: they all read the same
    // P_j, which one L2 then serves (the grid is a multiple of 8 units)
    const int xcd = (int)blockIdx.x & 7, jj = (int)blockIdx.x >> 3;
    const int unit = (jj / NT) * 8 + xcd, tv = jj % NT;
    const SegTable t = seg_table(a, C);
    if (unit >= nu) return;
    const int n = unit / H;
    const int k = __builtin_amdgcn_readlane(t.k, n);
    if (k <= 2) return;
    const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(wave_id());
    const int r16 = lane & 15, g = lane >> 4;
    // step j's operands for this wave's row blocks rb = w + r NW, as in the combine's state
    // rows: pa[r][q][e] = P_j[16 rb + r16][16 q + 4 g + e], da[r][e] = Delta_j[16 rb + 4 g + e]
    // [16 tv + r16], so step (q, e) contracts over keys 16 q + 4 g + e with S_j's same rows
    f32x4 pa[RBW][NQ], pn[RBW][NQ];
    f32x4 da[RBW], dn[RBW];
    auto load_step = [&](int j, f32x4 (&p)[RBW][NQ], f32x4 (&d)[RBW]) {
        const size_t bu = (size_t)(j - 1) * nu + unit;
        const float* P = a.ws.ptrans + bu * DK * DV;
        const float* Dl = a.ws.delta + bu * DK * DV;
#pragma unroll
        for (int r = 0; r < RBW; r++) {
            const int rb = w + r * NW;
#pragma unroll
            for (int q = 0; q < NQ; q++)
                p[r][q] = *reinterpret_cast<const f32x4*>(P + (size_t)(16 * rb + r16) * DK + 16 * q + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; e++) d[r][e] = Dl[(size_t)(16 * rb + 4 * g + e) * DV + 16 * tv + r16];
        }
    };
    // step j with its operands (pc, dc), loading step j + 1's into (px, dx) first: issued
    // unconditionally (the last step reloads its own), and kept ahead of the products, so
    // their latency overlaps the step and the wait counts stay exact
    auto step = [&](int j, f32x4 (&pc)[RBW][NQ], f32x4 (&dc)[RBW], f32x4 (&px)[RBW][NQ],
                    f32x4 (&dx)[RBW]) {
        load_step(min(j + 1, k - 2), px, dx);
        __builtin_amdgcn_sched_barrier(0);
        f32x4 sb[NQ];  // sb[q][e] = S_j[16 q + 4 g + e][16 tv + r16]
#pragma unroll
        for (int q = 0; q < NQ; q++) sb[q] = *reinterpret_cast<const f32x4*>(&slt[r16][16 * q + 4 * g]);
        __builtin_amdgcn_sched_barrier(0);
        f32x4 acc[RBW];
#pragma unroll
        for (int r = 0; r < RBW; r++) acc[r] = dc[r];
#pragma unroll
        for (int q = 0; q < NQ; q++)
#pragma unroll
            for (int e = 0; e < 4; e++)
#pragma unroll
                for (int r = 0; r < RBW; r++) acc[r] = MF::mma(pc[r][q][e], sb[q][e], acc[r]);
        __syncthreads();  // every wave has read S_j
        const size_t bn = (size_t)j * nu + unit;
        T* smt = reinterpret_cast<T*>(a.ws.smidt) + bn * DV * DK;
        float* sm = a.ws.smid + bn * DK * DV;
#pragma unroll
        for (int r = 0; r < RBW; r++) {
            const int rb = w + r * NW;
            float sv[4] = {acc[r][0], acc[r][1], acc[r][2], acc[r][3]};
            *reinterpret_cast<f32x4*>(&slt[r16][16 * rb + 4 * g]) = acc[r];
            store4<T>(smt + (size_t)(16 * tv + r16) * DK + 16 * rb + 4 * g, sv);
            if (j == k - 2)
#pragma unroll
                for (int e = 0; e < 4; e++) sm[(size_t)(16 * rb + 4 * g + e) * DV + 16 * tv + r16] = sv[e];
        }
        __syncthreads();  // S_{j+1} complete in LDS
    };
    load_step(1, pa, da);
    {  // S_1's column slice, 16-byte loads (4 columns of one key row each), stored transposed
        const float* s1 = a.ws.smid + (size_t)unit * DK * DV + 16 * tv;
        f32x4 x[DK * 16 / 4 / CB_THREADS];
#pragma unroll
        for (int it = 0; it < DK * 16 / 4 / CB_THREADS; it++) {
            const int p = (int)threadIdx.x + it * CB_THREADS;
            x[it] = *reinterpret_cast<const f32x4*>(s1 + (size_t)(p / 4) * DV + 4 * (p % 4));
        }
#pragma unroll
        for (int it = 0; it < DK * 16 / 4 / CB_THREADS; it++) {
            const int p = (int)threadIdx.x + it * CB_THREADS;
#pragma unroll
            for (int e = 0; e < 4; e++) slt[4 * (p % 4) + e][p / 4] = x[it][e];
        }
    }
    __syncthreads();
    for (int j = 1; j <= k - 2; j += 2) {  // two steps per pass: the operand sets alternate
        step(j, pa, da, pn, dn);
        if (j + 1 > k - 2) break;
        step(j + 1, pn, dn, pa, da);
    }
}

// Combine pass. Workgroups [0, n_seqs H d_k / 16): 16 state rows of a (sequence, head)
// whose sequence was split into k segments, S = P S_{k-1} + Delta with the last segment's
// P and Delta, on fp32 MFMA, written to its pool slot (none for a slot outside the pool).
// They come first so they run beside the rest. Then one workgroup per chunk of a later
// segment j (counted over the sequences, head-minor): O = O0 + L S_j on bf16 MFMA (O0 in
// fp32; L and S_j rounded to bf16, as the scan rounds Q_in and S for Q_in S), one wave per
// 16-token block, written to o.
// later-segment chunks of a call, at most (the grid's chunk part is H times this): a
// sequence of n chunks cut into k <= kmax has n - ceil(n seg_first_64(k) / 64) of them, and
// the share falls as k grows
inline int64_t seg_b_chunks_bound(int64_t max_chunks, int kmax) {
    return (max_chunks * (64 - seg_first_64(kmax)) + 63) / 64 + 1;
}
template <typename T, int DK, int DV, int C>
__global__ __launch_bounds__(CB_THREADS) void prefill_seg_combine_kernel(PrefillArgs a) {
    using MM = Mma<T>;
    using MF = Mma<float>;
    constexpr int KB = MM::KB, KPL = MM::KPL, NB = C / 16, NT = DV / 16;
    constexpr int V16 = 16 / (int)sizeof(T);  // elements per 16 bytes
    constexpr int LDT = DK + V16;  // S_j^T rows in LDS (16-byte padding)
    constexpr int LDO = DV + V16;  // output rows in LDS
    static_assert(NB == CB_THREADS / WAVE, "one wave per 16-token block");
    static_assert(DK % KB == 0 && DK % 16 == 0, "no key padding");
    static_assert(NB * 16 * LDO <= DV * LDT, "output rows reuse the S_j^T space");
    __shared__ __align__(16) T lds[DV * LDT];
    const int H = a.H, nu = a.n_seqs * H;
    const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(wave_id());
    const int r16 = lane & 15, g = lane >> 4;
    const SegTable t = seg_table(a, C);
    const int n_state = nu * (DK / 16);

    if ((int)blockIdx.x < n_state) {
        const int unit = (int)blockIdx.x / (DK / 16), rb = (int)blockIdx.x % (DK / 16);
        const int n = unit / H, h = unit - n * H;
        const int k = __builtin_amdgcn_readlane(t.k, n);
        if (k < 2) return;  // not split: stored by the scan
        const int slot = a.slots[n];
        if (slot < 0 || slot >= a.n_slots) return;
        const size_t bu = (size_t)(k - 2) * nu + unit;  // the last boundary
        const float* P = a.ws.ptrans + bu * DK * DV;
        const float* Sm = a.ws.smid + bu * DK * DV;
        const float* Dl = a.ws.delta + bu * DK * DV;
        float* S = a.state_pool + ((size_t)slot * H + h) * DK * DV;
        // A operand: lane (r16, g) holds P[16 rb + r16][16 q + 4 g + e] in pa[q][e], and the
        // B operand of step (q, e) the same key rows of S_{k-1}, so each step contracts over
        // keys 16 q + e + {0, 4, 8, 12}: all d_k keys once over the DK / 4 steps
        f32x4 pa[DK / 16];
#pragma unroll
        for (int q = 0; q < DK / 16; q++)
            pa[q] = *reinterpret_cast<const f32x4*>(P + (size_t)(16 * rb + r16) * DK + 16 * q + 4 * g);
        for (int tv = w; tv < NT; tv += CB_THREADS / WAVE) {
            f32x4 acc;
#pragma unroll
            for (int e = 0; e < 4; e++) acc[e] = Dl[(size_t)(16 * rb + 4 * g + e) * DV + 16 * tv + r16];
            float sb[DK / 4];
#pragma unroll
            for (int q = 0; q < DK / 16; q++)
#pragma unroll
                for (int e = 0; e < 4; e++)
                    sb[4 * q + e] = Sm[(size_t)(16 * q + 4 * g + e) * DV + 16 * tv + r16];
#pragma unroll
            for (int q = 0; q < DK / 16; q++)
#pragma unroll
                for (int e = 0; e < 4; e++) acc = MF::mma(pa[q][e], sb[4 * q + e], acc);
#pragma unroll
            for (int e = 0; e < 4; e++) S[(size_t)(16 * rb + 4 * g + e) * DV + 16 * tv + r16] = acc[e];
        }
        return;
    }
    const int id = (int)blockIdx.x - n_state;
    const int h = id % H, kc = id / H;
    const uint64_t m = __ballot(lane < a.n_seqs && t.pex <= kc && kc < t.pin);
    if (m == 0) return;
    const int n = __builtin_ctzll(m);
    const int c0 = __builtin_amdgcn_readlane(t.c0, n), c1 = __builtin_amdgcn_readlane(t.c1, n);
    const int k = __builtin_amdgcn_readlane(t.k, n);
    const int c = seg_bound(c0, c1, 1, k) + (kc - __builtin_amdgcn_readlane(t.pex, n));
    int j = 1;  // the chunk's segment
    while (j + 1 < k && seg_bound(c0, c1, j + 1, k) <= c) j++;
    const size_t u = (size_t)c * H + h;
    const float* o0 = reinterpret_cast<const float*>(a.ws.ut) + u * DV * C;
    const T* lb = reinterpret_cast<const T*>(a.ws.lbuf) + u * C * DK;
    const T* smt = reinterpret_cast<const T*>(a.ws.smidt) + ((size_t)(j - 1) * nu + n * H + h) * DV * DK;
    const int mb = w;
    f32x4 acc[NT];
#pragma unroll
    for (int tv = 0; tv < NT; tv++)
        acc[tv] = *reinterpret_cast<const f32x4*>(o0 + ((size_t)(tv * NB + mb) * 64 + lane) * 4);
    typename MM::frag al[DK / KB];
#pragma unroll
    for (int kb = 0; kb < DK / KB; kb++) al[kb] = MM::load(Frag<T>::ptr(lb, mb, kb, DK, lane));
    // S_j^T into LDS once for all four waves, 16 bytes per copy
    static_assert((DV * DK / V16) % CB_THREADS == 0, "S_j^T in whole 16-byte pieces");
#pragma unroll
    for (int it = 0; it < DV * DK / V16 / CB_THREADS; it++) {
        const int p = (int)threadIdx.x + it * CB_THREADS, row = p / (DK / V16), cv = p % (DK / V16);
        *reinterpret_cast<f32x4*>(&lds[row * LDT + cv * V16]) =
            *reinterpret_cast<const f32x4*>(smt + (size_t)row * DK + cv * V16);
    }
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < DK / KB; kb++)
#pragma unroll
        for (int tv = 0; tv < NT; tv++)
            acc[tv] = MM::mma(al[kb], MM::load(&lds[(16 * tv + r16) * LDT + kb * KB + g * KPL]), acc[tv]);
    __syncthreads();  // the S_j^T space now holds each wave's output rows
    T* ob = lds + mb * 16 * LDO;
#pragma unroll
    for (int tv = 0; tv < NT; tv++)
#pragma unroll
        for (int e = 0; e < 4; e++) ob[(4 * g + e) * LDO + 16 * tv + r16] = from_f32<T>(acc[tv][e]);
    asm volatile("" ::: "memory");  // LDS accesses of one wave complete in order
    const int tok0 = a.cu_seqlens[n] + (c - c0) * C;
    const int len = min(C, min(a.cu_seqlens[n + 1], a.total_tokens) - tok0);
    const int row = lane >> 2, i = mb * 16 + row;
    if (i < len && tok0 + i >= 0) {
        T* dst = reinterpret_cast<T*>(a.o) + ((size_t)(tok0 + i) * H + h) * DV;
#pragma unroll
        for (int q = 0; q < DV / 32; q++) {  // 4 lanes per row, 8 columns per piece
            const int col = ((lane & 3) + 4 * q) * 8;
            float v8[8];
            load8<T>(&ob[row * LDO + col], v8);
            store8<T>(dst + col, v8);
        }
    }
}

// =====================================================================================
// dispatch for one element type
// =====================================================================================
__global__ void seq_first_kernel(const int32_t* cu, int n_seqs, int C, int32_t* seq_first);

// nvb comes from scan_tiles, which never exceeds D / 16 (nor 4 for fp32), so the
// instantiated tile width always equals nvb (the ternaries only keep impossible
// combinations from being instantiated): the grid was sized for it, and the prep chose who
// forms U by it.
template <typename T, int D, int C, bool PERKEY, bool CKPT, bool QRAW>
void scan_launch_q(const PrefillArgs& a, int nvb, unsigned grid, hipStream_t s) {
    const dim3 block(ScanShape<C>::THREADS);
    constexpr int N8 = D >= 128 && sizeof(T) == 2 ? 8 : 1;  // see scan_tiles
    switch (nvb) {
        // 16-column tiles never read q themselves (PrefillArgs::q_raw)
        case 1: hipLaunchKernelGGL((prefill_scan_kernel<T, D, D, C, PERKEY, 1, CKPT, false>), dim3(grid), block, 0, s, a); break;
        case 2: hipLaunchKernelGGL((prefill_scan_kernel<T, D, D, C, PERKEY, D >= 32 ? 2 : 1, CKPT, QRAW>), dim3(grid), block, 0, s, a); break;
        case 4: hipLaunchKernelGGL((prefill_scan_kernel<T, D, D, C, PERKEY, D >= 64 ? 4 : 1, CKPT, QRAW>), dim3(grid), block, 0, s, a); break;
        default: hipLaunchKernelGGL((prefill_scan_kernel<T, D, D, C, PERKEY, N8, CKPT, QRAW>), dim3(grid), block, 0, s, a); break;
    }
}
template <typename T, int D, int C, bool PERKEY, bool CKPT>
void scan_launch(const PrefillArgs& a, int nvb, unsigned grid, hipStream_t s) {
    if (!PERKEY && a.q_raw) scan_launch_q<T, D, C, PERKEY, CKPT, !PERKEY>(a, nvb, grid, s);
    else scan_launch_q<T, D, C, PERKEY, CKPT, false>(a, nvb, grid, s);
}

template <typename T, int D, int C, bool PERKEY, bool CONV>
hipError_t prefill_prep_cfg(const PrefillArgs& a, hipStream_t s) {
    const size_t smem = sizeof(PrepSmem<T, D, D, C, PERKEY, CONV>);
    static_assert(sizeof(PrepSmem<T, D, D, C, PERKEY, CONV>) <= 160 * 1024,
                  "prep LDS over 160 KiB");
    auto prep = prefill_prep_kernel<T, D, D, C, PERKEY, CONV>;
    // dynamic LDS above 64 KiB must be allowed explicitly (idempotent, no library state);
    // done before the first launch so a refusal launches nothing
    hipError_t e = hipFuncSetAttribute((const void*)prep,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return e;
    }
    if (a.n_seqs > SEQ_INLINE_MAX)  // shorter lists: each wave forms the table itself
        hipLaunchKernelGGL(seq_first_kernel, dim3(1), dim3(256), 0, s, a.cu_seqlens, a.n_seqs,
                           C, a.ws.seq_first);
    const int64_t nchunk = a.ws.max_chunks;
    if (nchunk > 0)
        hipLaunchKernelGGL(prep, dim3((unsigned)((CONV ? nchunk : ((nchunk + 7) / 8) * 8) * a.H)),
                           dim3(PF_THREADS), smem, s, a);
    return hipGetLastError();
}

template <typename T, int D, int C, bool PERKEY>
hipError_t prefill_scan_cfg(const PrefillArgs& a, hipStream_t s) {
    const int units = a.n_seqs * a.H;
    if constexpr ((D == 128 || D == 64) && C == 64) {
        if (a.seg) {  // see seg_segments
            const int kmax = a.seg;
            const unsigned grid = (unsigned)(((kmax * units + 7) / 8) * 8 * (D / SCAN_BV));
            hipLaunchKernelGGL((prefill_scan_seg_kernel<T, D, C, PERKEY>), dim3(grid),
                               dim3(ScanShape<C>::THREADS), 0, s, a);
            if (kmax > 2)
                hipLaunchKernelGGL((prefill_seg_chain_kernel<T, D, D, C>), dim3((unsigned)(((units + 7) / 8) * 8 * (D / 16))),
                                   dim3(CB_THREADS), 0, s, a);
            const int64_t nb = seg_b_chunks_bound(a.ws.max_chunks, kmax) * a.H + (int64_t)units * (D / 16);
            hipLaunchKernelGGL((prefill_seg_combine_kernel<T, D, D, C>), dim3((unsigned)nb),
                               dim3(CB_THREADS), 0, s, a);
            return hipGetLastError();
        }
    }
    const int nvb = scan_tiles(a.dtype, units, D);
    const unsigned grid = (unsigned)(((units + 7) / 8) * 8 * (D / (SCAN_BV * nvb)));
    if (a.ckpt_cu != nullptr) scan_launch<T, D, C, PERKEY, true>(a, nvb, grid, s);
    else scan_launch<T, D, C, PERKEY, false>(a, nvb, grid, s);
    return hipGetLastError();
}

// Calls fn(D, C, PERKEY), each an integral constant, for the call's head dim, chunk size
// and gate kind.
template <typename Fn>
hipError_t prefill_dispatch(const PrefillArgs& a, Fn&& fn) {
    using std::integral_constant;
    auto gate = [&](auto D, auto C) {
        return a.gate == 1 ? fn(D, C, std::true_type{}) : fn(D, C, std::false_type{});
    };
    auto chunk = [&](auto D) {
        switch (a.chunk) {
            case 16: return gate(D, integral_constant<int, 16>{});
            case 32: return gate(D, integral_constant<int, 32>{});
            case 64: return gate(D, integral_constant<int, 64>{});
        }
        return hipErrorInvalidValue;
    };
    switch (a.dk) {
        case 16: return chunk(integral_constant<int, 16>{});
        case 32: return chunk(integral_constant<int, 32>{});
        case 64: return chunk(integral_constant<int, 64>{});
        case 128: return chunk(integral_constant<int, 128>{});
    }
    return hipErrorInvalidValue;
}

// prep (q, k, v given) followed by the scan
template <typename T>
hipError_t prefill_launch_typed(const PrefillArgs& a, hipStream_t s) {
    return prefill_dispatch(a, [&](auto D, auto C, auto PK) {
        hipError_t e = prefill_prep_cfg<T, D, C, PK, false>(a, s);
        return e != hipSuccess ? e : prefill_scan_cfg<T, D, C, PK>(a, s);
    });
}
template <typename T>
hipError_t prefill_scan_typed(const PrefillArgs& a, hipStream_t s) {
    return prefill_dispatch(a, [&](auto D, auto C, auto PK) {
        return prefill_scan_cfg<T, D, C, PK>(a, s);
    });
}
template <typename T>
hipError_t prefill_conv_prep_typed(const PrefillArgs& a, hipStream_t s) {
    return prefill_dispatch(a, [&](auto D, auto C, auto PK) {
        return prefill_prep_cfg<T, D, C, PK, true>(a, s);
    });
}

}  // namespace gdn
