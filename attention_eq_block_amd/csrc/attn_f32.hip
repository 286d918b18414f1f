// Eq. (1) of Nemotron-TwoTower (arXiv 2606.26493, section 2.1) for float32
// inputs: one wavefront per query row (b, s, h), lanes spread over head_dim,
// keys visited in order (prefix tokens through the page table, then the S
// block tokens) with an online softmax in float32. This path serves float32
// callers and small shapes; the bf16 MFMA path is the throughput path.
#include "tt_internal.h"

namespace tt {
namespace {

struct F32Args {
    const float* Q;
    long long qsb, qss, qsh;
    const float* Kc;
    const float* Vc;
    int page_size, num_pages, max_pages, Lmax;
    const int* page_table;
    const int* ctx_len;
    const float* Kd;
    const float* Vd;
    long long dsb, dss, dsh;
    float* O;
    long long osb, oss, osh;
    float* LSE;
    int B, S, Hq, Hkv, G;
    float scale;
};

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

template <int D>
__global__ __launch_bounds__(256) void attn_f32_kernel(F32Args a) {
    constexpr int E = D / 64;  // elements of head_dim per lane
    const int lane = threadIdx.x & 63;
    const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const long long n_rows = (long long)a.B * a.S * a.Hq;
    if (row >= n_rows) return;
    const int h = (int)(row % a.Hq);
    const int s = (int)((row / a.Hq) % a.S);
    const int b = (int)(row / ((long long)a.Hq * a.S));
    const int g = h / a.G;
    const int L = a.ctx_len ? clamp_len(a.ctx_len[b], a.Lmax) : 0;
    const int n = L + (a.Kd ? a.S : 0);

    float q[E], o[E];
    const float* qp = a.Q + b * a.qsb + s * a.qss + h * a.qsh + lane * E;
#pragma unroll
    for (int e = 0; e < E; ++e) { q[e] = qp[e]; o[e] = 0.f; }
    float m = -INFINITY, l = 0.f;
    for (int j = 0; j < n; ++j) {
        const float* kp;
        const float* vp;
        bool ok = true;
        if (j < L) {
            const int page = a.page_table[(long long)b * a.max_pages + j / a.page_size];
            ok = page >= 0 && page < a.num_pages;
            const long long off = (((long long)(ok ? page : 0) * a.Hkv + g) * a.page_size + j % a.page_size) * D;
            kp = a.Kc + off;
            vp = a.Vc + off;
        } else {
            const long long off = b * a.dsb + (long long)(j - L) * a.dss + g * a.dsh;
            kp = a.Kd + off;
            vp = a.Vd + off;
        }
        float k[E], v[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            k[e] = ok ? kp[lane * E + e] : 0.f;
            v[e] = ok ? vp[lane * E + e] : 0.f;
        }
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) part = __builtin_fmaf(q[e], k[e], part);
        const float sc = wave_sum(part) * a.scale;
        const float mn = fmaxf(m, sc);
        const float alpha = expf(m - mn);  // 0 when m = -inf
        const float p = expf(sc - mn);
        l = l * alpha + p;
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = __builtin_fmaf(p, v[e], o[e] * alpha);
        m = mn;
    }
    float* op = a.O + b * a.osb + s * a.oss + h * a.osh + lane * E;
    const float inv = n > 0 ? 1.f / l : 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) op[e] = o[e] * inv;
    if (a.LSE && lane == 0) a.LSE[((long long)b * a.Hq + h) * a.S + s] = n > 0 ? m + logf(l) : -INFINITY;
}

}  // namespace

tt_status launch_attn_f32(const tt_block_attn_params& p, hipStream_t s) {
    F32Args a{};
    a.Q = static_cast<const float*>(p.Q);
    a.qsb = p.q_stride_b; a.qss = p.q_stride_s; a.qsh = p.q_stride_h;
    a.Kc = static_cast<const float*>(p.Kctx);
    a.Vc = static_cast<const float*>(p.Vctx);
    a.page_size = p.page_size; a.num_pages = p.num_pages; a.max_pages = p.max_pages;
    const long long cap = (long long)p.max_pages * p.page_size;
    a.Lmax = (int)(p.max_ctx_len < cap ? p.max_ctx_len : cap);
    a.page_table = p.page_table;
    a.ctx_len = p.max_ctx_len > 0 ? p.ctx_len : nullptr;
    a.Kd = static_cast<const float*>(p.Kden);
    a.Vd = static_cast<const float*>(p.Vden);
    a.dsb = p.den_stride_b; a.dss = p.den_stride_s; a.dsh = p.den_stride_h;
    a.O = static_cast<float*>(p.O);
    a.osb = p.o_stride_b; a.oss = p.o_stride_s; a.osh = p.o_stride_h;
    a.LSE = p.LSE;
    a.B = p.B; a.S = p.S; a.Hq = p.Hq; a.Hkv = p.Hkv; a.G = p.Hq / p.Hkv;
    a.scale = p.softmax_scale;
    const long long rows = (long long)p.B * p.S * p.Hq;
    const dim3 grid((unsigned)((rows + 3) / 4));
    if (p.head_dim == 128)
        hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(256), 0, s, a);
    return hipGetLastError() == hipSuccess ? TT_OK : TT_ERR_HIP;
}

}  // namespace tt
