// Eq. (1) of Nemotron-TwoTower (arXiv 2606.26493, section 2.1) for float32
// inputs: one wavefront per query row (b, s, h). Keys are taken 64 at a time,
// one per lane: each lane computes its key's score against the query row
// (read from LDS as a broadcast) and copies its key's value row into the
// wave's LDS tile, one wave reduction per 64 keys gives the running max and
// sum (online softmax in float32), and the P.V product runs with lanes over
// head_dim, reading the weights and value rows from LDS. This path serves
// float32 callers and small shapes; the bf16 MFMA path is the throughput path.
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
    int* dbg;  // debug mode: TT_DEBUG_* bits of the out-of-range data read, or null
    int B, S, Hq, Hkv, G;
    float scale;
};

// x of another lane by a DPP pattern (`id` where the pattern names none or the
// row is masked off): a register move, no LDS round trip
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_move(float x, float id) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(__float_as_int(id), __float_as_int(x), CTRL, ROWS, 0xF, false));
}

// Sum and maximum over the 64 lanes of a wave (all active), in every lane: the
// running value within each row of 16 lanes by shifts of 1, 2, 4 and 8, then
// row 0's into row 1 and row 2's into row 3 (broadcast of lanes 15 and 47),
// then that of rows 0-1 into rows 2 and 3 (broadcast of lane 31); lane 63 then
// holds the result, which every lane reads.
template <class Op>
__device__ __forceinline__ float wave_reduce(float x, float id, Op op) {
    x = op(x, dpp_move<0x111, 0xF>(x, id));  // row_shr:1
    x = op(x, dpp_move<0x112, 0xF>(x, id));  // row_shr:2
    x = op(x, dpp_move<0x114, 0xF>(x, id));  // row_shr:4
    x = op(x, dpp_move<0x118, 0xF>(x, id));  // row_shr:8
    x = op(x, dpp_move<0x142, 0xA>(x, id));  // row_bcast:15, rows 1 and 3
    x = op(x, dpp_move<0x143, 0xC>(x, id));  // row_bcast:31, rows 2 and 3
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}
__device__ __forceinline__ float wave_sum(float x) {
    return wave_reduce(x, 0.f, [](float u, float v) { return u + v; });
}
__device__ __forceinline__ float wave_max(float x) {
    return wave_reduce(x, -INFINITY, [](float u, float v) { return fmaxf(u, v); });
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int D>
__global__ __launch_bounds__(256) void attn_f32_kernel(F32Args a) {
    constexpr int E = D / 64;  // elements of head_dim per lane in the P.V product
    __shared__ __attribute__((aligned(16))) float qs[4][D];
    // each wave's 64 value rows (padded pitch: the row-per-lane writes spread over the banks) and weights
    __shared__ __attribute__((aligned(16))) float vs[4][64][D + 4];
    __shared__ float ps[4][64];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const long long row = (long long)blockIdx.x * 4 + w;
    const long long n_rows = (long long)a.B * a.S * a.Hq;
    if (row >= n_rows) return;  // whole waves only: no barrier below
    const int h = (int)(row % a.Hq);
    const int s = (int)((row / a.Hq) % a.S);
    const int b = (int)(row / ((long long)a.Hq * a.S));
    const int g = h / a.G;
    const int L = a.ctx_len ? clamp_len(a.ctx_len[b], a.Lmax) : 0;
    if (a.dbg && a.ctx_len && lane == 0 && s == 0 && h == 0) {
        const int raw = a.ctx_len[b];
        if (raw < 0 || raw > a.Lmax) atomicOr(a.dbg, TT_DEBUG_CTX_LEN);
    }
    const int n = L + (a.Kd ? a.S : 0);
    if (a.dbg) {
        // debug mode: this wave's LDS slots start as NaN, so a read of one that no store of
        // this call filled reaches the output (the fences below order the fill first)
        const float qnan = __builtin_nanf("");
        for (int i = lane; i < D; i += 64) qs[w][i] = qnan;
        for (int r = 0; r < 64; ++r)
            for (int i = lane; i < D + 4; i += 64) vs[w][r][i] = qnan;
        ps[w][lane] = qnan;
    }

    // the query row, in this wave's LDS slot (read back as broadcasts)
    const float* qp = a.Q + b * a.qsb + s * a.qss + h * a.qsh;
#pragma unroll
    for (int e = 0; e < E; ++e) qs[w][lane * E + e] = qp[lane * E + e];
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    float o[E];
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = 0.f;
    float m = -INFINITY, l = 0.f;
    for (int j0 = 0; j0 < n; j0 += 64) {
        // this lane's key j (past the end: the last key again, weight 0)
        const int j = min(j0 + lane, n - 1);
        const float* kp;
        const float* vp;
        if (j < L) {
            // a page id outside the pool is clamped into it (wrong data, no fault)
            int page = a.page_table[(long long)b * a.max_pages + j / a.page_size];
            if (page < 0 || page >= a.num_pages) {
                if (a.dbg) atomicOr(a.dbg, TT_DEBUG_PAGE_ID);
                page = min(max(page, 0), a.num_pages - 1);
            }
            const long long off = (((long long)page * a.Hkv + g) * a.page_size + j % a.page_size) * D;
            kp = a.Kc + off;
            vp = a.Vc + off;
        } else {
            const long long off = b * a.dsb + (long long)(j - L) * a.dss + g * a.dsh;
            kp = a.Kd + off;
            vp = a.Vd + off;
        }
        // this lane's value row into the wave's LDS tile (its loads go out with the key row's)
#pragma unroll
        for (int d = 0; d < D; d += 4)
            *reinterpret_cast<f32x4*>(&vs[w][lane][d]) = *reinterpret_cast<const f32x4*>(vp + d);
        // score of key j: its row against the query row, 4 elements at a time
        float dot = 0.f;
#pragma unroll 8
        for (int d = 0; d < D; d += 4) {
            const f32x4 kv = *reinterpret_cast<const f32x4*>(kp + d);
            const f32x4 qv = *reinterpret_cast<const f32x4*>(&qs[w][d]);
            dot = __builtin_fmaf(kv[0], qv[0], dot);
            dot = __builtin_fmaf(kv[1], qv[1], dot);
            dot = __builtin_fmaf(kv[2], qv[2], dot);
            dot = __builtin_fmaf(kv[3], qv[3], dot);
        }
        const bool valid = j0 + lane < n;
        const float sc = valid ? dot * a.scale : -INFINITY;
        const float mn = fmaxf(m, wave_max(sc));
        const float alpha = expf(m - mn);  // 0 when m = -inf
        const float p = valid ? expf(sc - mn) : 0.f;
        l = l * alpha + wave_sum(p);
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] *= alpha;
        m = mn;
        // O += sum over the chunk's keys t of p_t * V_t, lanes over head_dim, from LDS
        ps[w][lane] = p;
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int nt = min(64, n - j0);
#pragma unroll 8
        for (int t = 0; t < nt; ++t) {
            const float pt = ps[w][t];
#pragma unroll
            for (int e = 0; e < E; ++e) o[e] = __builtin_fmaf(pt, vs[w][t][lane * E + e], o[e]);
        }
        // the next chunk rewrites the tile only after these reads
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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
    a.dbg = p.debug_flags;
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
