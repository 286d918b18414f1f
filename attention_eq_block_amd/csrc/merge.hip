// Log-sum-exp merge of partial attentions (tt_lse_merge). Attention over the
// concatenated key set of Eq. (1) (Nemotron-TwoTower, arXiv 2606.26493,
// section 2.1) equals the softmax-weighted combination of attentions over
// disjoint parts of it, each weighted by exp(lse_part - lse_total).
// One thread per (row, 4 consecutive head_dim elements); memory-bound.
#include "tt_internal.h"

namespace tt {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void lse_merge_kernel(int P, const float* __restrict__ O_parts,
                                                         const float* __restrict__ lse_parts, int B, int S,
                                                         int Hq, int d, void* O_out, int o_f32,
                                                         float* lse_out) {
    const int q = d / 4;
    const long long n_rows = (long long)B * S * Hq;
    const long long items = n_rows * q;
    for (long long it = (long long)blockIdx.x * blockDim.x + threadIdx.x; it < items;
         it += (long long)gridDim.x * blockDim.x) {
        const long long r = it / q;  // row index in [B][S][Hq] order
        const int c = (int)(it % q);
        const int h = (int)(r % Hq);
        const int s = (int)((r / Hq) % S);
        const int b = (int)(r / ((long long)Hq * S));
        const long long li = ((long long)b * Hq + h) * S + s;  // [B][Hq][S]
        const long long lstride = (long long)B * Hq * S;
        float M = -INFINITY;
        for (int p = 0; p < P; ++p) M = fmaxf(M, lse_parts[p * lstride + li]);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        float W = 0.f;
        if (M != -INFINITY) {
            for (int p = 0; p < P; ++p) {
                const float l = lse_parts[p * lstride + li];
                if (l == -INFINITY) continue;
                const float w = __expf(l - M);
                W += w;
                const f32x4 v = *reinterpret_cast<const f32x4*>(O_parts + ((long long)p * n_rows + r) * d + c * 4);
                acc += w * v;
            }
        }
        const float inv = W > 0.f ? 1.f / W : 0.f;
        const f32x4 o = acc * inv;
        if (o_f32)
            *reinterpret_cast<f32x4*>(static_cast<float*>(O_out) + r * d + c * 4) = o;
        else
            *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(O_out) + r * d + c * 4) = __builtin_convertvector(o, bf16x4);
        if (lse_out && c == 0) lse_out[li] = W > 0.f ? M + __logf(W) : -INFINITY;
    }
}

}  // namespace

tt_status launch_lse_merge(int P, const float* O_parts, const float* lse_parts, int B, int S, int Hq, int d,
                           void* O_out, int o_dtype, float* lse_out, hipStream_t s) {
    const long long items = (long long)B * S * Hq * (d / 4);
    if (items == 0) return TT_OK;
    long long blocks = (items + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(lse_merge_kernel, dim3((unsigned)blocks), dim3(256), 0, s, P, O_parts, lse_parts, B, S,
                       Hq, d, O_out, o_dtype == TT_F32 ? 1 : 0, lse_out);
    return hipGetLastError() == hipSuccess ? TT_OK : TT_ERR_HIP;
}

}  // namespace tt
