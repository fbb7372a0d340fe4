// Prefill front end: per-sequence chunk table (device-side, no host synchronisation),
// workspace carving and dispatch to the element-type instantiations.
#include <algorithm>

#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_scan_bf16(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_scan_f32(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_conv_prep_bf16(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_conv_prep_f32(const PrefillArgs& a, hipStream_t s);

// seq_first[n] = sum_{s < n} ceil(len_s / C), n = 0..n_seqs (one workgroup, tiled scan).
__global__ __launch_bounds__(256) void seq_first_kernel(const int32_t* cu, int n_seqs, int C,
                                                        int32_t* seq_first) {
    __shared__ int32_t part[256];
    __shared__ int32_t carry;
    if (threadIdx.x == 0) carry = 0;
    __syncthreads();
    for (int base = 0; base < n_seqs; base += 256) {
        const int n = base + (int)threadIdx.x;
        int cnt = 0;
        if (n < n_seqs) {
            const int len = max(0, cu[n + 1] - cu[n]);
            cnt = (len + C - 1) / C;
        }
        part[threadIdx.x] = cnt;
        __syncthreads();
        // inclusive Hillis-Steele scan over 256 entries
        for (int off = 1; off < 256; off <<= 1) {
            int v = threadIdx.x >= (unsigned)off ? part[threadIdx.x - off] : 0;
            __syncthreads();
            part[threadIdx.x] += v;
            __syncthreads();
        }
        if (n < n_seqs) seq_first[n] = carry + part[threadIdx.x] - cnt;
        __syncthreads();
        if (threadIdx.x == 255) carry += part[255];
        __syncthreads();
    }
    if (threadIdx.x == 0) seq_first[n_seqs] = carry;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t prefill_ws_layout(int dtype, int H, int dk, int dv, int chunk, int n_seqs,
                         int total_tokens, void* base, PrefillWs* out) {
    const size_t e = dtype == 1 ? 2 : 4;
    const int cp = prefill_cp(dtype, chunk);
    const int dkp = prefill_dkp(dtype, dk);
    // upper bound on the chunk count: sum_s ceil(len_s / C) <= (T + n (C - 1)) / C
    const int64_t max_chunks =
        ((int64_t)total_tokens + (int64_t)n_seqs * (chunk - 1)) / chunk;
    const size_t units = (size_t)max_chunks * H;
    size_t off = 0;
    const size_t o_seq = off; off = align256(off + sizeof(int32_t) * (size_t)(n_seqs + 1));
    const size_t o_w = off;   off = align256(off + units * chunk * dkp * e);
    const size_t o_q = off;   off = align256(off + units * chunk * dkp * e);
    const size_t o_k = off;   off = align256(off + units * dk * cp * e);
    const size_t o_m = off;   off = align256(off + units * chunk * cp * e);
    // U (fp32) when the prep forms it; otherwise, in the same space, (R - I) diag(beta),
    // beta, (conv-fused prefill only; the plain prefill reads v itself) v after the
    // convolution and (raw-q scan only) the output row factors
    const size_t s_r = align256(units * chunk * cp * e);
    const size_t s_b = align256(units * chunk * 4);
    const size_t s_v = align256(units * chunk * dv * e);
    const size_t s_q = align256(units * chunk * 4);
    const size_t o_u = off;
    off = align256(off + std::max(units * dv * chunk * 4, s_r + s_b + s_v + s_q));
    const size_t o_d = off;   off = align256(off + units * dk * 4);
    // segmented scan: L per unit, and four d_k x d_v states per (segment boundary, sequence,
    // head): three in fp32, one (transposed) in the element type
    const int kseg = seg_segments(dtype, H, dk, dv, chunk, n_seqs, total_tokens);
    const bool seg = kseg != 0;
    const size_t sh = (size_t)(seg ? kseg - 1 : 0) * n_seqs * H * dk * dv;
    const size_t o_l = off;   if (seg) off = align256(off + units * chunk * dkp * e);
    const size_t o_sm = off;  if (seg) off = align256(off + sh * 4);
    const size_t o_st = off;  if (seg) off = align256(off + sh * e);
    const size_t o_p = off;   if (seg) off = align256(off + sh * 4);
    const size_t o_dl = off;  if (seg) off = align256(off + sh * 4);
    const size_t o_x = off;   off = align256(off + 256 * 4);
    if (out != nullptr) {
        char* b = static_cast<char*>(base);
        out->chunk_info = nullptr;
        out->seq_first = reinterpret_cast<int32_t*>(b + o_seq);
        out->wneg = b + o_w;
        out->qin = b + o_q;
        out->kgt = b + o_k;
        out->mmat = b + o_m;
        out->ut = b + o_u;
        out->rr = b + o_u;
        out->beta = reinterpret_cast<float*>(b + o_u + s_r);
        out->vbuf = b + o_u + s_r + s_b;
        out->qs = reinterpret_cast<float*>(b + o_u + s_r + s_b + s_v);
        out->decay = reinterpret_cast<float*>(b + o_d);
        out->lbuf = seg ? b + o_l : nullptr;
        out->smid = seg ? reinterpret_cast<float*>(b + o_sm) : nullptr;
        out->smidt = seg ? b + o_st : nullptr;
        out->ptrans = seg ? reinterpret_cast<float*>(b + o_p) : nullptr;
        out->delta = seg ? reinterpret_cast<float*>(b + o_dl) : nullptr;
        out->dump = b + o_x;
        out->max_chunks = max_chunks;
    }
    return off;
}

hipError_t launch_prefill(const PrefillArgs& args, hipStream_t s) {
    // zero tokens still defines the final states (initial state, or zero), so only an
    // empty sequence list is a no-op
    if (args.n_seqs == 0) return hipSuccess;
    PrefillArgs a = args;
    a.u_ws = scan_tiles(a.dtype, (int64_t)a.n_seqs * a.H, a.dv) == 1;
    a.q_raw = a.gate == 0 && a.conv_width == 0 && !a.u_ws;
    // the workspace holds the segmented-scan sections, for this K, exactly when
    // seg_segments returns K
    a.seg = a.ckpt_cu == nullptr && a.ws.lbuf != nullptr
                ? seg_segments(a.dtype, a.H, a.dk, a.dv, a.chunk, a.n_seqs, a.total_tokens)
                : 0;
    (void)hipGetLastError();  // report only errors raised by this call's launches
    const bool b16 = a.dtype == 1;
    if (a.conv_width == 0) return b16 ? launch_prefill_bf16(a, s) : launch_prefill_f32(a, s);
    // conv-fused: prep forms q, k, v from x; the conv history is advanced only after every
    // prep workgroup has read the old one (same stream, next launch)
    hipError_t e = b16 ? launch_prefill_conv_prep_bf16(a, s) : launch_prefill_conv_prep_f32(a, s);
    if (e == hipSuccess) e = b16 ? launch_prefill_scan_bf16(a, s) : launch_prefill_scan_f32(a, s);
    if (e == hipSuccess && a.conv_state != nullptr) e = launch_conv_state_update(a, s);
    return e;
}

}  // namespace gdn
