// Causal depthwise short convolution (width <= 4) followed by SiLU, over packed varlen
// sequences, writing q|k|v planes.
//
// Page: [LA-Infra] "深度解析线性注意力机制演进与 AI Infra 实现", section "去掉分母引入卷积"
// (per channel, fixed weights over the current and previous tokens, weight column
// width-1 on the current token, then SiLU; zero history at a sequence start) and
// "vLLM中Decode的实现" (one convolution over the concatenated q|k|v channels equals three).
//
// HBM-bound elementwise pass: each thread produces 8 adjacent channels (one 16-byte access
// for bf16) of CONV_TT consecutive tokens, so the width-1 history rows it reads besides its
// own tokens add (width-1)/CONV_TT to the read traffic. Rows are kept in registers in the
// input type and widened to fp32 when used.
#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {

constexpr int CONV_THREADS = 256;

// Each thread produces 8 adjacent channels of CONV_TT consecutive tokens: the weights are
// read once (float4 per channel), each x row once, and the window slides in registers.
constexpr int CONV_TT = 16;

// 8 consecutive elements kept in their storage type
template <typename T> struct Row8;
template <> struct Row8<bf16> {
    bf16x8 v;
    __device__ __forceinline__ void load(const bf16* p) { v = *reinterpret_cast<const bf16x8*>(p); }
    __device__ __forceinline__ void zero() { v = Mma<bf16>::zero(); }
    __device__ __forceinline__ float operator[](int i) const { return (float)v[i]; }
};
template <> struct Row8<float> {
    f32x4 lo, hi;
    __device__ __forceinline__ void load(const float* p) {
        lo = *reinterpret_cast<const f32x4*>(p);
        hi = *reinterpret_cast<const f32x4*>(p + 4);
    }
    __device__ __forceinline__ void zero() { lo = zero4(); hi = zero4(); }
    __device__ __forceinline__ float operator[](int i) const { return i < 4 ? lo[i] : hi[i - 4]; }
};

template <typename T, int W>
__global__ __launch_bounds__(CONV_THREADS) void conv1d_silu_kernel(ConvArgs a) {
    const int groups = a.channels / 8;
    const int tgroups = (a.total_tokens + CONV_TT - 1) / CONV_TT;
    const int64_t idx = (int64_t)blockIdx.x * CONV_THREADS + threadIdx.x;
    if (idx >= (int64_t)tgroups * groups) return;
    const int tg = (int)(idx / groups);
    const int c0 = (int)(idx - (int64_t)tg * groups) * 8;
    const int t0 = tg * CONV_TT;
    // sequence of token t0: last n with cu_seqlens[n] <= t0 (binary search)
    int lo = 0, hi = a.n_seqs;
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (a.cu_seqlens[mid] <= t0) lo = mid; else hi = mid;
    }
    int start = a.cu_seqlens[lo];
    int next = a.cu_seqlens[lo + 1];
    float wv[8][4];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        if constexpr (W == 4) {
            f32x4 w4 = *reinterpret_cast<const f32x4*>(a.w + (size_t)(c0 + i) * 4);
            wv[i][0] = w4[0]; wv[i][1] = w4[1]; wv[i][2] = w4[2]; wv[i][3] = w4[3];
        } else {
#pragma unroll
            for (int j = 0; j < W; j++) wv[i][j] = a.w[(size_t)(c0 + i) * W + j];
        }
    }
    const T* x = reinterpret_cast<const T*>(a.x);
    // rows t0-(W-1) .. t0+CONV_TT-1, zero outside [0, total_tokens)
    constexpr int NR = CONV_TT + W - 1;
    Row8<T> xr[NR];
#pragma unroll
    for (int r = 0; r < NR; r++) {
        const int src = t0 - (W - 1) + r;
        if (src >= 0 && src < a.total_tokens) xr[r].load(x + (size_t)src * a.channels + c0);
        else xr[r].zero();
    }
    const int pc = a.channels / a.planes;
    const int plane = c0 / pc;
    T* ybase = reinterpret_cast<T*>(a.y) + (size_t)plane * a.total_tokens * pc + (c0 - plane * pc);
#pragma unroll
    for (int tt = 0; tt < CONV_TT; tt++) {
        const int t = t0 + tt;
        if (t >= a.total_tokens) break;
        while (t >= next && lo + 1 < a.n_seqs) {  // crossed into the next sequence
            lo++;
            start = a.cu_seqlens[lo];
            next = a.cu_seqlens[lo + 1];
        }
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < W; j++) {
            const int src = t - (W - 1) + j;
            const bool keep = src >= start;  // zero history before the sequence start
#pragma unroll
            for (int i = 0; i < 8; i++) acc[i] = fmaf(wv[i][j], keep ? xr[tt + j][i] : 0.f, acc[i]);
        }
#pragma unroll
        for (int i = 0; i < 8; i++) acc[i] = silu_f32(acc[i]);
        T* dst = ybase + (size_t)t * pc;
        if constexpr (sizeof(T) == 2) {  // output rows are streamed: non-temporal stores
            bf16x8 v;
#pragma unroll
            for (int i = 0; i < 8; i++) v[i] = (bf16)acc[i];
            __builtin_nontemporal_store(v, reinterpret_cast<bf16x8*>(dst));
        } else {
            __builtin_nontemporal_store(f32x4{acc[0], acc[1], acc[2], acc[3]},
                                        reinterpret_cast<f32x4*>(dst));
            __builtin_nontemporal_store(f32x4{acc[4], acc[5], acc[6], acc[7]},
                                        reinterpret_cast<f32x4*>(dst + 4));
        }
    }
}

template <typename T>
static hipError_t conv_launch(const ConvArgs& a, hipStream_t s) {
    const int64_t work = (int64_t)((a.total_tokens + CONV_TT - 1) / CONV_TT) * (a.channels / 8);
    dim3 grid((unsigned)((work + CONV_THREADS - 1) / CONV_THREADS)), block(CONV_THREADS);
    switch (a.width) {
        case 2: hipLaunchKernelGGL((conv1d_silu_kernel<T, 2>), grid, block, 0, s, a); break;
        case 3: hipLaunchKernelGGL((conv1d_silu_kernel<T, 3>), grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL((conv1d_silu_kernel<T, 4>), grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_conv1d(const ConvArgs& a, hipStream_t s) {
    if (a.total_tokens == 0 || a.n_seqs == 0) return hipSuccess;
    (void)hipGetLastError();  // report only errors raised by this call's launches
    return a.dtype == 1 ? conv_launch<bf16>(a, s) : conv_launch<float>(a, s);
}

// One thread per (sequence, channel): the new history is the last W-1 rows of the
// sequence's raw projection, where a row before the sequence start is the old history's
// entry for it (zero without one). Row r of the new history holds token end-(W-1)+r, so
// column 0 stays the oldest, as the decode step expects.
template <typename T>
__global__ __launch_bounds__(256) void conv_state_update_kernel(PrefillArgs a) {
    const int XC = 3 * a.H * a.dk;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)a.n_seqs * XC) return;
    const int n = (int)(idx / XC), ch = (int)(idx - (int64_t)n * XC);
    const int slot = a.slots[n];
    if (slot < 0 || slot >= a.n_slots) return;
    const int W = a.conv_width;
    const int s0 = a.cu_seqlens[n], s1 = a.cu_seqlens[n + 1];
    const bool hist = a.has_init != nullptr && a.has_init[n] != 0;
    T* cs = reinterpret_cast<T*>(a.conv_state) + ((size_t)slot * XC + ch) * (W - 1);
    const T* x = reinterpret_cast<const T*>(a.x);
    T old[3], nw[3];
#pragma unroll
    for (int j = 0; j < 3; j++) old[j] = (hist && j < W - 1) ? cs[j] : from_f32<T>(0.f);
    const int len = s1 - s0;
#pragma unroll
    for (int j = 0; j < 3; j++) {
        // only the W-1 entries that are stored: for j >= W-1 the row would be s1 or later,
        // past the sequence (and past x for the last one)
        const int r = s1 - (W - 1) + j;
        // (rows outside [0, total_tokens), possible only with cu_seqlens that break the
        // contract, read as zero; the old-history index is selected, never computed)
        const int oi = j + len;
        if (j >= W - 1) nw[j] = from_f32<T>(0.f);
        else if (r >= s0) nw[j] = (r >= 0 && r < a.total_tokens) ? x[(size_t)r * XC + ch]
                                                                 : from_f32<T>(0.f);
        else nw[j] = oi == 0 ? old[0] : oi == 1 ? old[1] : (oi == 2 && W - 1 > 2) ? old[2]
                                                                             : from_f32<T>(0.f);
    }
#pragma unroll
    for (int j = 0; j < 3; j++)
        if (j < W - 1) cs[j] = nw[j];
}

hipError_t launch_conv_state_update(const PrefillArgs& a, hipStream_t s) {
    const int64_t work = (int64_t)a.n_seqs * 3 * a.H * a.dk;
    if (work == 0) return hipSuccess;
    const dim3 grid((unsigned)((work + 255) / 256)), block(256);
    if (a.dtype == 1) hipLaunchKernelGGL(conv_state_update_kernel<bf16>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(conv_state_update_kernel<float>, grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace gdn
