// One-token recurrent decode over a slot-indexed fp32 state pool (dense), and the DeltaLog
// variant (dense base + append log, merged every M steps).
//
// Pages: [LA-Infra] "深度解析线性注意力机制演进与 AI Infra 实现", sections "GDN：增加遗忘门",
// "KDA实现逻辑概述" (per-token step list), App. 2 (L2 norm); [Handbook] "线性注意力与混合架构的推理",
// "投机解码与 PD 分离" (fixed slots, batched kernel addresses states by slot index);
// [DeltaLog] "DeltaLog：延迟物化递归状态以加速线性注意力解码" reading notes, §1.2 (the step is
// bound by the state stream, about 0.5 flop/byte), §2.1-2.4 (base + log, Algorithm 1,
// Eqs. 4-7), §2.6 (one writer for the shared log metadata).
//
// Design (MI355X): one 512-thread workgroup owns one (request, head) state, d_k x d_v fp32
// (64 KiB at d = 128). Each thread holds 4 adjacent value columns of d_k / (512 / (d_v/4))
// rows in registers, so the state is read from HBM once, both column reductions
// (vhat = Sbar^T k and Sbar^T q) come from the same registers, and the update is written
// back once with 16-byte coalesced, non-temporal accesses along d_v. Reductions:
// xor-shuffles inside a wave, one LDS exchange across the 8 waves. With B*H workgroups
// (4096 at B = 128, H = 32) every CU keeps several 64 KiB streams in flight. Because one workgroup covers the whole
// value range, the DeltaLog key-side replay coefficients are computed once per
// (request, head) in-workgroup and a single thread is the one writer of K_log, Lambda_log,
// lbar and L — no separate replay-prep launch and no scratch buffer.
#include "gdn.h"
#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {

constexpr float L2_EPS = 1e-6f;
constexpr int DEC_THREADS = 256;        // DeltaLog kernels
constexpr int DENSE_THREADS = 512;      // dense decode: more state rows in flight per workgroup
constexpr int DL_MAXLOG = 16;  // M - 1 <= 16

template <int DK, int DV, int NT = DEC_THREADS>
struct DecGeom {
    static constexpr int TPR = DV / 4;                 // threads per state row
    static constexpr int RPP = NT / TPR;               // rows per pass
    static constexpr int NP = (DK + RPP - 1) / RPP;    // passes
    static constexpr int NWAVE = NT / WAVE;
    // lanes of a wave that hold the same column group
    static constexpr int ROWS_PER_WAVE = WAVE / TPR;
};

// The state is touched exactly once per step: streamed with non-temporal loads and stores
// so it does not displace other lines from the caches (measured: the state update runs
// closer to the HBM rate this way).
__device__ __forceinline__ f32x4 stream_load(const float* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}
__device__ __forceinline__ void stream_store(float* p, f32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
}

// Shared prologue: stage k, q (fp32, optionally L2-normalised), v, and per-key decay in
// LDS; every wave computes the norms itself to avoid an extra barrier.
template <typename T, int DK, int DV>
struct DecSmem {
    float k[DK];
    float q[DK];
    float v[DV];
    float gk[DK];
    float red_v[DecGeom<DK, DV, DENSE_THREADS>::NWAVE][DV];
    float red_q[DecGeom<DK, DV, DENSE_THREADS>::NWAVE][DV];
    float r[DV];
};

template <int DK>
__device__ __forceinline__ void kq_norms(const float* ks, const float* qs, float& ik, float& iq,
                                         float& kq, bool l2norm) {
    // each wave reduces the full d_k vectors (DK <= 128: at most two values per lane)
    const int l = lane_id();
    float sk = 0.f, sq = 0.f, skq = 0.f;
    for (int i = l; i < DK; i += WAVE) {
        float a = ks[i], b = qs[i];
        sk += a * a;
        sq += b * b;
        skq += a * b;
    }
    sk = group_sum<WAVE>(sk);
    sq = group_sum<WAVE>(sq);
    skq = group_sum<WAVE>(skq);
    if (l2norm) {
        ik = rsqrtf(sk + L2_EPS);
        iq = rsqrtf(sq + L2_EPS);
    } else {
        ik = 1.f;
        iq = 1.f;
    }
    kq = skq * ik * iq;
}

// One token of the gated delta rule on the state slice this thread holds in registers
// (st[p] = S[r0 + p RPP][4 cg .. 4 cg + 3]):
//   Sbar = Diag(decay) S;  vhat = Sbar^T k;  r = beta (v - vhat);  S <- Sbar + k r^T;
//   o = scale S^T q = scale (Sbar^T q + (k . q) r).
// k, q, v (fp32, unnormalised) and gk (e^{g} per key channel) are staged in LDS; ik, iq are
// the L2 scales of k and q (1 without normalisation) and kq = (k . q) ik iq. Both column
// reductions come from the same registers: xor-shuffles inside a wave, then one LDS
// exchange across the waves. Returns the output column `tid` (meaningful for tid < d_v).
// Ends with every thread past the exchange, so the caller may restage LDS afterwards only
// behind another barrier.
template <int DK, int DV, bool PERKEY, int NP>
__device__ __forceinline__ float token_update(f32x4 (&st)[NP], const float* k, const float* q,
                                              const float* v, const float* gk, float alpha,
                                              float beta, float ik, float iq, float kq,
                                              float scale, float (*red_v)[DV],
                                              float (*red_q)[DV], float* rbuf) {
    using G = DecGeom<DK, DV, DENSE_THREADS>;
    static_assert(NP == G::NP, "state registers per thread");
    const int tid = threadIdx.x;
    const int cg = tid % G::TPR;
    const int r0 = tid / G::TPR;
    // decay and the two column reductions from the same registers
    float pv[4] = {0.f, 0.f, 0.f, 0.f}, pq[4] = {0.f, 0.f, 0.f, 0.f};
    float kr[G::NP];
#pragma unroll
    for (int p = 0; p < G::NP; p++) {
        const int r = r0 + p * G::RPP;
        if (r < DK) {
            const float dec = PERKEY ? gk[r] : alpha;
            const float kk = k[r] * ik, qq = q[r] * iq;
            kr[p] = kk;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                float s = st[p][i] * dec;
                st[p][i] = s;
                pv[i] += s * kk;
                pq[i] += s * qq;
            }
        }
    }
    // reduce across the lanes of this wave that share the column group
#pragma unroll
    for (int off = G::TPR; off < WAVE; off <<= 1) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            pv[i] += __shfl_xor(pv[i], off, WAVE);
            pq[i] += __shfl_xor(pq[i], off, WAVE);
        }
    }
    const int w = wave_id();
    if (lane_id() < G::TPR) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            red_v[w][cg * 4 + i] = pv[i];
            red_q[w][cg * 4 + i] = pq[i];
        }
    }
    lds_barrier();
    float out = 0.f;
    if (tid < DV) {
        float vh = 0.f, sh = 0.f;
#pragma unroll
        for (int ww = 0; ww < G::NWAVE; ww++) {
            vh += red_v[ww][tid];
            sh += red_q[ww][tid];
        }
        const float r = beta * (v[tid] - vh);
        rbuf[tid] = r;
        out = scale * (sh + kq * r);
    }
    lds_barrier();
    float rr[4];
#pragma unroll
    for (int i = 0; i < 4; i++) rr[i] = rbuf[cg * 4 + i];
#pragma unroll
    for (int p = 0; p < G::NP; p++) {
        const int r = r0 + p * G::RPP;
        if (r < DK) {
#pragma unroll
            for (int i = 0; i < 4; i++) st[p][i] += kr[p] * rr[i];
        }
    }
    return out;
}

template <typename T, int DK, int DV, bool PERKEY>
__global__ __launch_bounds__(DENSE_THREADS) void decode_kernel(DecodeArgs a) {
    using G = DecGeom<DK, DV, DENSE_THREADS>;
    __shared__ DecSmem<T, DK, DV> sm;
    const int tid = threadIdx.x;
    const int H = a.H;
    const int bh = blockIdx.x;
    const int b = bh / H, h = bh - (bh / H) * H;
    const int slot = a.slots[b];
    T* o = reinterpret_cast<T*>(a.o) + (size_t)bh * DV;
    if (slot < 0 || slot >= a.n_slots) {
        if (tid < DV / 4) {
            float z[4] = {0.f, 0.f, 0.f, 0.f};
            store4<T>(o + tid * 4, z);
        }
        return;
    }
    const int cg = tid % G::TPR;
    const int r0 = tid / G::TPR;
    float* S = a.pool + ((size_t)slot * H + h) * DK * DV;

    // the token's vectors first (their staging and the norms then overlap the state read),
    // then the state stream
    const T* qp = reinterpret_cast<const T*>(a.q) + (size_t)bh * DK;
    const T* kp = reinterpret_cast<const T*>(a.k) + (size_t)bh * DK;
    const T* vp = reinterpret_cast<const T*>(a.v) + (size_t)bh * DV;
    float kx = 0.f, qx = 0.f, gx = 0.f, vx = 0.f;
    if (tid < DK) {
        kx = to_f32(kp[tid]);
        qx = to_f32(qp[tid]);
        if (PERKEY) gx = a.g[(size_t)bh * DK + tid];
    }
    if (tid < DV) vx = to_f32(vp[tid]);
    const float beta = a.beta[bh];
    const float gs = PERKEY ? 0.f : a.g[bh];
    f32x4 st[G::NP];
#pragma unroll
    for (int p = 0; p < G::NP; p++) {
        const int r = r0 + p * G::RPP;
        if (r < DK) st[p] = stream_load(S + (size_t)r * DV + cg * 4);
    }
    if (tid < DK) {
        sm.k[tid] = kx;
        sm.q[tid] = qx;
        if (PERKEY) sm.gk[tid] = __expf(gx);
    }
    if (tid < DV) sm.v[tid] = vx;
    const float alpha = PERKEY ? 1.f : __expf(gs);
    lds_barrier();

    float ik, iq, kq;
    kq_norms<DK>(sm.k, sm.q, ik, iq, kq, a.l2norm != 0);
    const float out = token_update<DK, DV, PERKEY>(st, sm.k, sm.q, sm.v, sm.gk, alpha, beta, ik,
                                                   iq, kq, a.scale, sm.red_v, sm.red_q, sm.r);
    if (tid < DV) o[tid] = from_f32<T>(out);
#pragma unroll
    for (int p = 0; p < G::NP; p++) {
        const int r = r0 + p * G::RPP;
        if (r < DK) stream_store(S + (size_t)r * DV + cg * 4, st[p]);
    }
}

// Multi-token verify step of speculative decoding. Each request feeds n_pos tokens (the
// confirmed token and the drafts); the state after every position is stored in that
// position's slot, and the round starts from the slot of column num_accepted - 1 of the
// previous round, so a rejected draft is rolled back by choosing a column, with no copy
// ([LA-Infra] "推测解码：验证后如何恢复状态"; [Handbook] "投机解码与 PD 分离").
// One workgroup per (request, head) keeps the state in registers across the positions:
// one 64 KiB read and n_pos 64 KiB writes per head at d = 128.
constexpr int SPEC_MAX_POS = GDN_SPEC_MAX_POS;

// The reduction buffers are static; the n_pos positions' vectors live in dynamic LDS sized
// by the call (at d = 128 and 4 positions 15 KiB in all, so 4 workgroups share a CU):
//   k[P][DK], q[P][DK], v[P][DV], gk[P][DK] (per-key gate only), alpha[P], beta[P]
template <int DK, int DV>
struct SpecSmem {
    float red_v[DecGeom<DK, DV, DENSE_THREADS>::NWAVE][DV];
    float red_q[DecGeom<DK, DV, DENSE_THREADS>::NWAVE][DV];
    float r[DV];
};
template <int DK, int DV, bool PERKEY>
constexpr size_t spec_dyn_bytes(int P) {
    return (size_t)P * ((PERKEY ? 3 : 2) * DK + DV + 2) * sizeof(float);
}
// the largest call (d = 128, per-key gate, the most positions the ABI accepts) stays within
// the 64 KiB a launch gets without raising its LDS limit
static_assert(spec_dyn_bytes<128, 128, true>(SPEC_MAX_POS) + sizeof(SpecSmem<128, 128>) <=
                  64 * 1024,
              "spec-decode LDS at the maximum position count");

template <typename T, int DK, int DV, bool PERKEY>
__global__ __launch_bounds__(DENSE_THREADS) void spec_decode_kernel(DecodeArgs a) {
    using G = DecGeom<DK, DV, DENSE_THREADS>;
    __shared__ SpecSmem<DK, DV> sm;
    extern __shared__ __align__(16) float spec_dyn[];
    const int tid = threadIdx.x;
    const int H = a.H, P = a.n_pos;
    float* ks = spec_dyn;
    float* qs = ks + P * DK;
    float* vs = qs + P * DK;
    float* gks = vs + P * DV;
    float* alphas = gks + (PERKEY ? P * DK : 0);
    float* betas = alphas + P;
    const int bh = blockIdx.x;
    const int b = bh / H, h = bh - (bh / H) * H;
    const int32_t* row = a.slots + (size_t)b * P;
    const int col = a.num_accepted[b] - 1;
    const int slot0 = (col >= 0 && col < P) ? row[col] : -1;
    // o[b, j, h, :] lives at o + ((b P + j) H + h) d_v
    T* o = reinterpret_cast<T*>(a.o) + ((size_t)b * P * H + h) * DV;
    if (slot0 < 0 || slot0 >= a.n_slots) {  // inactive request: zero outputs, no state access
        for (int i = tid; i < P * (DV / 4); i += DENSE_THREADS) {
            float z[4] = {0.f, 0.f, 0.f, 0.f};
            store4<T>(o + (size_t)(i / (DV / 4)) * H * DV + (i % (DV / 4)) * 4, z);
        }
        return;
    }
    const int cg = tid % G::TPR;
    const int r0 = tid / G::TPR;
    // all positions' vectors are staged before the state stream completes
    const T* qp = reinterpret_cast<const T*>(a.q);
    const T* kp = reinterpret_cast<const T*>(a.k);
    const T* vp = reinterpret_cast<const T*>(a.v);
    for (int i = tid; i < P * DK; i += DENSE_THREADS) {
        const int j = i / DK, c = i - j * DK;
        const size_t t = ((size_t)b * P + j) * H + h;
        ks[i] = to_f32(kp[t * DK + c]);
        qs[i] = to_f32(qp[t * DK + c]);
        if (PERKEY) gks[i] = __expf(a.g[t * DK + c]);
    }
    for (int i = tid; i < P * DV; i += DENSE_THREADS) {
        const int j = i / DV, c = i - j * DV;
        vs[i] = to_f32(vp[(((size_t)b * P + j) * H + h) * DV + c]);
    }
    if (tid < P) {
        const size_t t = ((size_t)b * P + tid) * H + h;
        betas[tid] = a.beta[t];
        alphas[tid] = PERKEY ? 1.f : __expf(a.g[t]);
    }
    const float* S0 = a.pool + ((size_t)slot0 * H + h) * DK * DV;
    f32x4 st[G::NP];
#pragma unroll
    for (int p = 0; p < G::NP; p++) {
        const int r = r0 + p * G::RPP;
        if (r < DK) st[p] = stream_load(S0 + (size_t)r * DV + cg * 4);
    }
    lds_barrier();
    for (int j = 0; j < P; j++) {
        float ik, iq, kq;
        const float* kj = ks + j * DK;
        const float* qj = qs + j * DK;
        kq_norms<DK>(kj, qj, ik, iq, kq, a.l2norm != 0);
        const float out = token_update<DK, DV, PERKEY>(st, kj, qj, vs + j * DV, gks + j * DK,
                                                       alphas[j], betas[j], ik, iq, kq,
                                                       a.scale, sm.red_v, sm.red_q, sm.r);
        if (tid < DV) o[(size_t)j * H * DV + tid] = from_f32<T>(out);
        const int sj = row[j];
        if (sj >= 0 && sj < a.n_slots) {
            float* Sj = a.pool + ((size_t)sj * H + h) * DK * DV;
#pragma unroll
            for (int p = 0; p < G::NP; p++) {
                const int r = r0 + p * G::RPP;
                if (r < DK) stream_store(Sj + (size_t)r * DV + cg * 4, st[p]);
            }
        }
    }
}

// Fused KDA decode step ([LA-Infra] "KDA实现逻辑概述", "vLLM中Decode的实现", "去掉分母引入卷积"):
// the workgroup of (request, head) first runs the causal short convolution of the head's
// 3 d channels (q, k, v planes) from the slot's conv state (the width - 1 previous inputs
// before the convolution), applies SiLU and shifts the window by the new input; then forms
// the gates in the kernel,
//   forget_log = lower_bound * sigmoid(e^{A_log} (forget_b + dt_bias)),  beta = sigmoid(logit),
// and runs the per-key token update on the convolved q, k, v (q, k L2-normalised). Each conv
// channel belongs to exactly one head, so the window update has a single writer.
template <typename T, int DK, int DV, int W>
__global__ __launch_bounds__(DENSE_THREADS) void fused_decode_kernel(FusedDecodeArgs a) {
    using G = DecGeom<DK, DV, DENSE_THREADS>;
    static_assert(DK == DV && 3 * DK <= DENSE_THREADS, "one conv channel per thread");
    __shared__ DecSmem<T, DK, DV> sm;
    const int tid = threadIdx.x;
    const int H = a.H;
    const int bh = blockIdx.x;
    const int b = bh / H, h = bh - (bh / H) * H;
    const int slot = a.slots[b];
    T* o = reinterpret_cast<T*>(a.o) + (size_t)bh * DV;
    if (slot < 0 || slot >= a.n_slots) {  // inactive row: zero output, no state access
        if (tid < DV / 4) {
            float z[4] = {0.f, 0.f, 0.f, 0.f};
            store4<T>(o + tid * 4, z);
        }
        return;
    }
    const size_t CH = (size_t)3 * H * DK;
    const int plane = tid / DK, i = tid - plane * DK;
    const size_t c = (size_t)plane * H * DK + (size_t)h * DK + i;
    const bool conv = tid < 3 * DK;
    T* cs = reinterpret_cast<T*>(a.conv_state) + ((size_t)slot * CH + c) * (W - 1);
    // convolution and gate inputs first, then the state stream
    T old[W - 1];
    T xv = from_f32<T>(0.f);
    float wv[W];
    if (conv) {
#pragma unroll
        for (int j = 0; j < W - 1; j++) old[j] = cs[j];
        xv = reinterpret_cast<const T*>(a.x)[(size_t)b * CH + c];
#pragma unroll
        for (int j = 0; j < W; j++) wv[j] = a.conv_w[c * W + j];
    }
    float xg = 0.f;
    if (tid < DK) xg = a.forget_b[(size_t)bh * DK + tid] + a.dt_bias[(size_t)h * DK + tid];
    const float logit = a.write_logit[bh];
    const float ea = __expf(a.A_log[h]);
    const int cg = tid % G::TPR;
    const int r0 = tid / G::TPR;
    float* S = a.pool + ((size_t)slot * H + h) * DK * DV;
    f32x4 st[G::NP];
#pragma unroll
    for (int p = 0; p < G::NP; p++) {
        const int r = r0 + p * G::RPP;
        if (r < DK) st[p] = stream_load(S + (size_t)r * DV + cg * 4);
    }
    if (conv) {
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < W - 1; j++) acc += wv[j] * to_f32(old[j]);
        acc += wv[W - 1] * to_f32(xv);
        const float y = silu_f32(acc);
#pragma unroll
        for (int j = 0; j + 1 < W - 1; j++) cs[j] = old[j + 1];
        cs[W - 2] = xv;
        float* dst = plane == 0 ? sm.q : (plane == 1 ? sm.k : sm.v);
        dst[i] = y;
    }
    if (tid < DK) {
        const float fl = a.lower_bound / (1.f + __expf(-ea * xg));
        sm.gk[tid] = __expf(fl);
    }
    const float beta = 1.f / (1.f + __expf(-logit));
    lds_barrier();

    float ik, iq, kq;
    kq_norms<DK>(sm.k, sm.q, ik, iq, kq, a.l2norm != 0);
    const float out = token_update<DK, DV, true>(st, sm.k, sm.q, sm.v, sm.gk, 1.f, beta, ik, iq,
                                                 kq, a.scale, sm.red_v, sm.red_q, sm.r);
    if (tid < DV) o[tid] = from_f32<T>(out);
#pragma unroll
    for (int p = 0; p < G::NP; p++) {
        const int r = r0 + p * G::RPP;
        if (r < DK) stream_store(S + (size_t)r * DV + cg * 4, st[p]);
    }
}

// ------------------------------------------------------------------------------ DeltaLog
template <int DK, int DV, bool PERKEY>
struct DlSmem {
    float k[DK];
    float q[DK];
    float v[DV];
    float klog[DL_MAXLOG][DK];     // logged keys; per-key gate: replaced by the decayed keys
    float lamk[PERKEY ? DL_MAXLOG : 1][DK];  // per-key Lambda_i
    float lp[PERKEY ? DK : 1];     // per-key lbar' = lbar + g
    float dk[PERKEY ? DK : 1];     // per-key e^{lbar'}
    alignas(16) float ulog[DL_MAXLOG][DV];
    float lam[DL_MAXLOG];
    float ck[DL_MAXLOG];  // e^{lp - Lambda_i} (k . K_i)
    float cq[DL_MAXLOG];  // e^{lp - Lambda_i} (q . K_i)
    float wl[DL_MAXLOG];  // e^{lp - Lambda_i}
    float red_v[DecGeom<DK, DV, DENSE_THREADS>::NWAVE][DV];
    float red_q[DecGeom<DK, DV, DENSE_THREADS>::NWAVE][DV];
    float b[DV];
};

// PERKEY: KDA-style per-key-channel decay. lbar and every Lambda_i are d_k wide, D(x) is
// diag(e^x) over key rows, so the replay of entry i weighs key channel c by
// e^{lbar'_c - Lambda_{i,c}}: the logged key is replaced in LDS by that decayed key, and the
// replay coefficients and the merge then use it unchanged ([DeltaLog] §2.7, the KDA row).
template <typename T, int DK, int DV, bool PERKEY>
__global__ __launch_bounds__(DENSE_THREADS) void deltalog_kernel(DeltaLogArgs a) {
    using G = DecGeom<DK, DV, DENSE_THREADS>;
    __shared__ DlSmem<DK, DV, PERKEY> sm;
    constexpr int DL = PERKEY ? DK : 1;  // width of lbar and Lambda
    const int tid = threadIdx.x;
    const int H = a.H;
    const int bh = blockIdx.x;
    const int b = bh / H, h = bh - (bh / H) * H;
    const int slot = a.slots[b];
    T* o = reinterpret_cast<T*>(a.o) + (size_t)bh * DV;
    if (slot < 0 || slot >= a.n_slots) {
        if (tid < DV / 4) {
            float z[4] = {0.f, 0.f, 0.f, 0.f};
            store4<T>(o + tid * 4, z);
        }
        return;
    }
    const int C = a.M - 1;
    const size_t sh = (size_t)slot * H + h;
    const int cg = tid % G::TPR;
    const int r0 = tid / G::TPR;
    float* S = a.base + sh * DK * DV;
    // clamp so that corrupted metadata can never index past the log buffers
    const int L = min(max(a.len[sh], 0), C);
    // The log (at most 16 x (d_k bf16 + d_v fp32)) is requested before the base stream, in
    // 16-byte pieces (8 keys or 4 values per thread), so its staging and the key-side replay
    // do not wait behind the 64 KiB base read.
    const uint16_t* kl = a.klog + sh * C * DK;
    const float* ul = a.ulog + sh * C * DV;
    const float* lamp = a.lamlog + sh * C * DL;
    constexpr int KPIECES = DL_MAXLOG * DK / 8, UPIECES = DL_MAXLOG * DV / 4;
    static_assert(KPIECES <= DENSE_THREADS && UPIECES <= DENSE_THREADS &&
                  DL_MAXLOG * DK / 4 <= DENSE_THREADS, "one piece per thread");
    const bool kpiece = tid * 8 < L * DK, upiece = tid * 4 < L * DV;
    const bool lpiece = PERKEY && tid * 4 < L * DK;
    bf16x8 kraw;
    f32x4 uraw, lraw;
    if (kpiece) kraw = *reinterpret_cast<const bf16x8*>(kl + tid * 8);
    if (upiece) uraw = *reinterpret_cast<const f32x4*>(ul + tid * 4);
    if (lpiece) lraw = *reinterpret_cast<const f32x4*>(lamp + tid * 4);
    f32x4 st[G::NP];
#pragma unroll
    for (int p = 0; p < G::NP; p++) {
        const int r = r0 + p * G::RPP;
        if (r < DK) st[p] = stream_load(S + (size_t)r * DV + cg * 4);
    }
    // Algorithm 1: accumulate the decay first
    const float lp = PERKEY ? 0.f : a.lbar[sh] + a.g[bh];
    if (PERKEY && tid < DK) {
        const float x = a.lbar[sh * DK + tid] + a.g[(size_t)bh * DK + tid];
        sm.lp[tid] = x;
        sm.dk[tid] = __expf(x);
    }
    const T* qp = reinterpret_cast<const T*>(a.q) + (size_t)bh * DK;
    const T* kp = reinterpret_cast<const T*>(a.k) + (size_t)bh * DK;
    const T* vp = reinterpret_cast<const T*>(a.v) + (size_t)bh * DV;
    if (tid < DK) {
        sm.k[tid] = to_f32(kp[tid]);
        sm.q[tid] = to_f32(qp[tid]);
    }
    if (tid < DV) sm.v[tid] = to_f32(vp[tid]);
    if (kpiece) {
        const int e = tid * 8 / DK, c0 = tid * 8 % DK;
#pragma unroll
        for (int i = 0; i < 8; i++) sm.klog[e][c0 + i] = (float)kraw[i];
    }
    if (upiece) {
        const int e = tid * 4 / DV, c0 = tid * 4 % DV;
        *reinterpret_cast<f32x4*>(&sm.ulog[e][c0]) = uraw;
    }
    if (lpiece) {
        const int e = tid * 4 / DK, c0 = tid * 4 % DK;
        *reinterpret_cast<f32x4*>(&sm.lamk[e][c0]) = lraw;
    }
    if (!PERKEY && tid < L) {
        float lam = a.lamlog[sh * C + tid];
        sm.lam[tid] = lam;
        sm.wl[tid] = __expf(lp - lam);
    }
    const float beta = a.beta[bh];
    lds_barrier();

    float ik, iq, kq;
    kq_norms<DK>(sm.k, sm.q, ik, iq, kq, a.l2norm != 0);
    // key-side replay coefficients, one wave per log entry (strided)
    {
        const int w = wave_id(), l = lane_id();
        for (int e = w; e < L; e += G::NWAVE) {
            float sk = 0.f, sq = 0.f;
            for (int i = l; i < DK; i += WAVE) {
                float ke = sm.klog[e][i];
                if (PERKEY) {  // decayed key, kept for the merge
                    ke *= __expf(sm.lp[i] - sm.lamk[e][i]);
                    sm.klog[e][i] = ke;
                }
                sk += sm.k[i] * ke;
                sq += sm.q[i] * ke;
            }
            sk = group_sum<WAVE>(sk);
            sq = group_sum<WAVE>(sq);
            if (l == 0) {
                sm.ck[e] = (PERKEY ? 1.f : sm.wl[e]) * sk * ik;
                sm.cq[e] = (PERKEY ? 1.f : sm.wl[e]) * sq * iq;
            }
        }
    }
    // Merge steps (uniform across the workgroup: L is per (slot, head)), scalar gate: the
    // log's part of the new base, sum_e w_e K_e U_e^T over this thread's rows and columns,
    // does not depend on the base, so it is formed here while the base stream is still in
    // flight; after the base arrives the merge is the dense update plus this sum (B = 512,
    // M = 8: cycle average 234.6 -> 231.0 us). The per-key gate keeps the sum after the base
    // reduction (its decayed keys come from the replay loop; done here, its appends slowed).
    const bool merging = L >= C;
    f32x4 lsum[PERKEY ? 1 : G::NP];
    if constexpr (!PERKEY) {
        if (merging) {
#pragma unroll
            for (int p = 0; p < G::NP; p++) lsum[p] = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int e = 0; e < L; e++) {
                const f32x4 ue = *reinterpret_cast<const f32x4*>(&sm.ulog[e][cg * 4]);
                const float we = sm.wl[e];
#pragma unroll
                for (int p = 0; p < G::NP; p++) {
                    const int r = r0 + p * G::RPP;
                    if (r < DK) {
                        const float c = we * sm.klog[e][r];
#pragma unroll
                        for (int i = 0; i < 4; i++) lsum[p][i] += c * ue[i];
                    }
                }
            }
        }
    }
    // base reads (undecayed base; the scalar factor e^{lp} is applied after the reduction,
    // a per-key factor with the key row)
    float pv[4] = {0.f, 0.f, 0.f, 0.f}, pq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < G::NP; p++) {
        const int r = r0 + p * G::RPP;
        if (r < DK) {
            const float dr = PERKEY ? sm.dk[r] : 1.f;
            const float kk = sm.k[r] * ik * dr, qq = sm.q[r] * iq * dr;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                pv[i] += st[p][i] * kk;
                pq[i] += st[p][i] * qq;
            }
        }
    }
#pragma unroll
    for (int off = G::TPR; off < WAVE; off <<= 1) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            pv[i] += __shfl_xor(pv[i], off, WAVE);
            pq[i] += __shfl_xor(pq[i], off, WAVE);
        }
    }
    {
        const int w = wave_id();
        if (lane_id() < G::TPR) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                sm.red_v[w][cg * 4 + i] = pv[i];
                sm.red_q[w][cg * 4 + i] = pq[i];
            }
        }
    }
    lds_barrier();
    const float dec = PERKEY ? 1.f : __expf(lp);
    if (tid < DV) {
        float vh = 0.f, shq = 0.f;
#pragma unroll
        for (int ww = 0; ww < G::NWAVE; ww++) {
            vh += sm.red_v[ww][tid];
            shq += sm.red_q[ww][tid];
        }
        vh *= dec;
        shq *= dec;
        for (int e = 0; e < L; e++) {
            vh += sm.ck[e] * sm.ulog[e][tid];
            shq += sm.cq[e] * sm.ulog[e][tid];
        }
        const float bb = beta * (sm.v[tid] - vh);
        sm.b[tid] = bb;
        o[tid] = from_f32<T>(a.scale * (shq + kq * bb));
    }
    if (L < C) {
        // append: the base is not written; one value entry, and a single writer for the
        // shared key entry and metadata of this (slot, head)
        lds_barrier();
        if (tid < DV) a.ulog[(sh * C + L) * DV + tid] = sm.b[tid];
        if (tid < DK) {
            bf16 kb = (bf16)(sm.k[tid] * ik);
            a.klog[(sh * C + L) * DK + tid] = __builtin_bit_cast(uint16_t, kb);
        }
        if (PERKEY) {
            if (tid < DK) {
                a.lamlog[(sh * C + L) * DK + tid] = sm.lp[tid];
                a.lbar[sh * DK + tid] = sm.lp[tid];
            }
        } else if (tid == 0) {
            a.lamlog[sh * C + L] = lp;
            a.lbar[sh] = lp;
        }
        if (tid == 0) a.len[sh] = L + 1;
        return;
    }
    // merge (Eq. 6): fold the log and the current update into the base, clear the log
    lds_barrier();
    float bb[4];
#pragma unroll
    for (int i = 0; i < 4; i++) bb[i] = sm.b[cg * 4 + i];
#pragma unroll
    for (int p = 0; p < G::NP; p++) {
        const int r = r0 + p * G::RPP;
        if (r < DK) {
            const float kk = sm.k[r] * ik;
            const float dr = PERKEY ? sm.dk[r] : dec;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                st[p][i] = st[p][i] * dr + kk * bb[i];
                if constexpr (!PERKEY) st[p][i] += lsum[p][i];
            }
        }
    }
    if constexpr (PERKEY) {
        // entry-outer: each entry's 4 value columns of this thread are read from LDS once
        // and applied to all of the thread's rows (klog holds the decayed keys)
        for (int e = 0; e < L; e++) {
            const f32x4 ue = *reinterpret_cast<const f32x4*>(&sm.ulog[e][cg * 4]);
#pragma unroll
            for (int p = 0; p < G::NP; p++) {
                const int r = r0 + p * G::RPP;
                if (r < DK) {
                    const float c = sm.klog[e][r];
#pragma unroll
                    for (int i = 0; i < 4; i++) st[p][i] += c * ue[i];
                }
            }
        }
    }
#pragma unroll
    for (int p = 0; p < G::NP; p++) {
        const int r = r0 + p * G::RPP;
        if (r < DK) stream_store(S + (size_t)r * DV + cg * 4, st[p]);
    }
    if (tid < DL) a.lbar[sh * DL + tid] = 0.f;
    if (tid == 0) a.len[sh] = 0;
}

// reset (mode 0) or materialize (mode 1) the listed slots; grid = n * H
template <int DK, int DV, bool PERKEY>
__global__ __launch_bounds__(DEC_THREADS) void deltalog_maint_kernel(DeltaLogArgs a, int mode) {
    using G = DecGeom<DK, DV>;
    constexpr int DL = PERKEY ? DK : 1;
    __shared__ float klog[DL_MAXLOG][DK];  // per key: the decayed keys
    __shared__ float ulog[DL_MAXLOG][DV];
    __shared__ float wl[DL_MAXLOG];
    __shared__ float dk[PERKEY ? DK : 1];
    const int tid = threadIdx.x;
    const int H = a.H;
    const int n = blockIdx.x / H, h = blockIdx.x % H;
    const int slot = a.slots[n];
    if (slot < 0 || slot >= a.n_slots) return;
    const size_t sh = (size_t)slot * H + h;
    if (mode == 1) {
        const int C = a.M - 1;
        const int L = min(max(a.len[sh], 0), C);
        const float* lb = a.lbar + sh * DL;
        const uint16_t* kl = a.klog + sh * C * DK;
        const float* ul = a.ulog + sh * C * DV;
        const float* lam = a.lamlog + sh * C * DL;
        for (int i = tid; i < L * DK; i += DEC_THREADS) {
            uint32_t bits = (uint32_t)kl[i] << 16;
            float kv = __builtin_bit_cast(float, bits);
            if (PERKEY) kv *= __expf(lb[i % DK] - lam[i]);
            klog[i / DK][i % DK] = kv;
        }
        for (int i = tid; i < L * DV; i += DEC_THREADS) ulog[i / DV][i % DV] = ul[i];
        if (!PERKEY && tid < L) wl[tid] = __expf(lb[0] - lam[tid]);
        if (PERKEY && tid < DK) dk[tid] = __expf(lb[tid]);
        lds_barrier();
        const float dec = PERKEY ? 1.f : __expf(lb[0]);
        const int cg = tid % G::TPR;
        const int r0 = tid / G::TPR;
        float* S = a.base + sh * DK * DV;
#pragma unroll
        for (int p = 0; p < G::NP; p++) {
            const int r = r0 + p * G::RPP;
            if (r < DK) {
                f32x4 s = *reinterpret_cast<const f32x4*>(S + (size_t)r * DV + cg * 4);
                const float dr = PERKEY ? dk[r] : dec;
#pragma unroll
                for (int i = 0; i < 4; i++) s[i] *= dr;
                for (int e = 0; e < L; e++) {
                    const float we = (PERKEY ? 1.f : wl[e]) * klog[e][r];
#pragma unroll
                    for (int i = 0; i < 4; i++) s[i] += we * ulog[e][cg * 4 + i];
                }
                *reinterpret_cast<f32x4*>(S + (size_t)r * DV + cg * 4) = s;
            }
        }
        lds_barrier();
    }
    if (tid < DL) a.lbar[sh * DL + tid] = 0.f;
    if (tid == 0) a.len[sh] = 0;
}

// ------------------------------------------------------------------------------- launch
template <typename T, int D>
static hipError_t dec_dispatch_gate(const DecodeArgs& a, hipStream_t s) {
    dim3 grid((unsigned)(a.batch * a.H)), block(DENSE_THREADS);
    if (a.num_accepted != nullptr) {
        const size_t dyn_pk = spec_dyn_bytes<D, D, true>(a.n_pos);
        const size_t dyn_sc = spec_dyn_bytes<D, D, false>(a.n_pos);
        if (a.gate == 1)
            hipLaunchKernelGGL((spec_decode_kernel<T, D, D, true>), grid, block, dyn_pk, s, a);
        else
            hipLaunchKernelGGL((spec_decode_kernel<T, D, D, false>), grid, block, dyn_sc, s, a);
    } else if (a.gate == 1) {
        hipLaunchKernelGGL((decode_kernel<T, D, D, true>), grid, block, 0, s, a);
    } else {
        hipLaunchKernelGGL((decode_kernel<T, D, D, false>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

template <typename T>
static hipError_t dec_dispatch_dim(const DecodeArgs& a, hipStream_t s) {
    switch (a.dk) {
        case 16: return dec_dispatch_gate<T, 16>(a, s);
        case 32: return dec_dispatch_gate<T, 32>(a, s);
        case 64: return dec_dispatch_gate<T, 64>(a, s);
        case 128: return dec_dispatch_gate<T, 128>(a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
    if (a.batch == 0) return hipSuccess;
    (void)hipGetLastError();  // report only errors raised by this call's launches
    return a.dtype == 1 ? dec_dispatch_dim<bf16>(a, s) : dec_dispatch_dim<float>(a, s);
}

template <typename T, int D>
static hipError_t fused_dispatch_width(const FusedDecodeArgs& a, hipStream_t s) {
    dim3 grid((unsigned)(a.batch * a.H)), block(DENSE_THREADS);
    switch (a.width) {
        case 2: hipLaunchKernelGGL((fused_decode_kernel<T, D, D, 2>), grid, block, 0, s, a); break;
        case 3: hipLaunchKernelGGL((fused_decode_kernel<T, D, D, 3>), grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL((fused_decode_kernel<T, D, D, 4>), grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T>
static hipError_t fused_dispatch_dim(const FusedDecodeArgs& a, hipStream_t s) {
    switch (a.dk) {
        case 16: return fused_dispatch_width<T, 16>(a, s);
        case 32: return fused_dispatch_width<T, 32>(a, s);
        case 64: return fused_dispatch_width<T, 64>(a, s);
        case 128: return fused_dispatch_width<T, 128>(a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_fused_decode(const FusedDecodeArgs& a, hipStream_t s) {
    if (a.batch == 0) return hipSuccess;
    (void)hipGetLastError();  // report only errors raised by this call's launches
    return a.dtype == 1 ? fused_dispatch_dim<bf16>(a, s) : fused_dispatch_dim<float>(a, s);
}

template <typename T, int D>
static hipError_t dl_launch(const DeltaLogArgs& a, hipStream_t s) {
    dim3 grid((unsigned)(a.batch * a.H)), block(DENSE_THREADS);
    if (a.gate == 1)
        hipLaunchKernelGGL((deltalog_kernel<T, D, D, true>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((deltalog_kernel<T, D, D, false>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <typename T>
static hipError_t dl_dispatch_dim(const DeltaLogArgs& a, hipStream_t s) {
    switch (a.dk) {
        case 16: return dl_launch<T, 16>(a, s);
        case 32: return dl_launch<T, 32>(a, s);
        case 64: return dl_launch<T, 64>(a, s);
        case 128: return dl_launch<T, 128>(a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_deltalog(const DeltaLogArgs& a, hipStream_t s) {
    if (a.batch == 0) return hipSuccess;
    (void)hipGetLastError();  // report only errors raised by this call's launches
    return a.dtype == 1 ? dl_dispatch_dim<bf16>(a, s) : dl_dispatch_dim<float>(a, s);
}

template <int D>
static hipError_t dlm_launch(const DeltaLogArgs& a, int mode, hipStream_t s) {
    dim3 grid((unsigned)(a.batch * a.H)), block(DEC_THREADS);
    if (a.gate == 1)
        hipLaunchKernelGGL((deltalog_maint_kernel<D, D, true>), grid, block, 0, s, a, mode);
    else
        hipLaunchKernelGGL((deltalog_maint_kernel<D, D, false>), grid, block, 0, s, a, mode);
    return hipGetLastError();
}

hipError_t launch_deltalog_maint(const DeltaLogArgs& a, int mode, hipStream_t s) {
    if (a.batch == 0) return hipSuccess;
    (void)hipGetLastError();  // report only errors raised by this call's launches
    switch (a.dk) {
        case 16: return dlm_launch<16>(a, mode, s);
        case 32: return dlm_launch<32>(a, mode, s);
        case 64: return dlm_launch<64>(a, mode, s);
        case 128: return dlm_launch<128>(a, mode, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdn
