// ConfidenceSample (Nemotron-TwoTower, arXiv 2606.26493, section 2.2
// "Sampling", Algorithm 2): one step of confidence unmasking.
//
// Kernel 1 (vocab_reduce): one pass over the logits of every MASKED row
// (unmasked rows are never read), gridded over rows x vocabulary splits. Each
// thread streams 16-byte chunks and keeps (max, first index of the max,
// sum of exp2((x - max) * log2(e)/temperature)); triples merge exactly across
// threads and splits, ties at the max going to the lower index.
// Kernel 2 (unmask_select): one wavefront per sequence, one lane per block
// position: confidence = 1/sum, then the commit rule -- every position above
// gamma if there are at least ceil(M/steps_left) of them, else the
// ceil(M/steps_left) most confident (ties to the lower position).
// Stochastic variant (the sampler's temperature argument, section 2.2
// "Sampling"), kernel 1b (sample_locate): a row with uniform u draws from
// softmax(x / temperature) by inverse transform sampling. The split masses of
// kernel 1 locate the split in which the cumulative sum passes u * Z; one
// workgroup re-reads only that split, each thread a contiguous run of it, and a
// workgroup scan of the run sums names the thread that walks its run again to
// the first element whose cumulative sum passes. The drawn token's probability
// replaces the greedy confidence in kernel 2.
// The masked-diffusion loss L_MD (Eq. (4)) runs vocab_reduce at temperature 1
// and a one-workgroup finish (nll_finish): lse - x[target] per masked row and
// their mean.
#include <limits.h>

#include "tt_internal.h"

namespace tt {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

struct Triple {
    float m;
    int a;
    float z;
    float pad;
};

struct Drawn {
    int a;
    float conf;
};

struct UArgs {
    const void* logits;
    long long stride;
    const uint8_t* mask_in;
    uint8_t* mask_out;
    int* tokens;
    float* conf;
    int* num_masked;
    Triple* part;  // [n_vsplit][B*S]
    const float* uniforms;  // [B*S] or null (greedy)
    Drawn* drawn;           // [B*S] when sampling
    int B, S, V, n_vsplit, steps_left;
    float gamma, c;  // c = log2(e) / temperature
};

__device__ __forceinline__ void combine(float& m, int& a, float& z, float m2, int a2, float z2, float c) {
    const float M = fmaxf(m, m2);
    float zz = 0.f;
    if (M != -INFINITY) {
        if (m != -INFINITY) zz += z * __builtin_amdgcn_exp2f((m - M) * c);
        if (m2 != -INFINITY) zz += z2 * __builtin_amdgcn_exp2f((m2 - M) * c);
    }
    a = m > m2 ? a : (m2 > m ? a2 : min(a, a2));
    m = M;
    z = zz;
}

// fold 8 consecutive logits starting at index v into (m, a, z)
__device__ __forceinline__ void fold8(const float (&x)[8], int v, float& m, int& a, float& z, float c) {
    float cm = x[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) cm = fmaxf(cm, x[k]);
    if (cm > m) {
        if (m != -INFINITY) z *= __builtin_amdgcn_exp2f((m - cm) * c);
        int k = 7;
#pragma unroll
        for (int kk = 7; kk >= 0; --kk) if (x[kk] == cm) k = kk;
        a = v + k;
        m = cm;
    }
    if (m != -INFINITY) {
        const float mc = m * c;
#pragma unroll
        for (int k = 0; k < 8; ++k) z += __builtin_amdgcn_exp2f(__builtin_fmaf(x[k], c, -mc));
    }
}

__device__ __forceinline__ void unpack(const u32x4& r, float (&x)[8]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        x[2 * k] = __uint_as_float(r[k] << 16);
        x[2 * k + 1] = __uint_as_float(r[k] & 0xffff0000u);
    }
}

// Element k of a row, widened to float.
template <bool BF16>
__device__ __forceinline__ float elem(const void* row, int k) {
    if (BF16) return __uint_as_float((unsigned)static_cast<const uint16_t*>(row)[k] << 16);
    return static_cast<const float*>(row)[k];
}

// Fold elements [lo, hi) (hi - lo <= 8) of a row as one padded chunk.
template <bool BF16>
__device__ __forceinline__ void fold_scalar(const void* row, int lo, int hi, float& m, int& a, float& z, float c) {
    float f[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) f[k] = lo + k < hi ? elem<BF16>(row, lo + k) : -INFINITY;
    fold8(f, lo, m, a, z, c);
}

// A row is cut as: a head of a0 < 8 elements up to the first 16-byte boundary,
// nfull aligned chunks of 8 elements, and a tail of fewer than 8. Split k of the
// grid takes an equal share of the chunks; split 0 also takes the head and the
// last split the tail. Each thread visits its elements in increasing index
// order, so the strict max update keeps the lowest index among its ties.
template <bool BF16>
__global__ __launch_bounds__(256) void vocab_reduce(UArgs a) {
    const int row = blockIdx.x;
    const int split = blockIdx.y;
    if (!a.mask_in[row]) return;
    constexpr int ES = BF16 ? 2 : 4;
    const char* rp = static_cast<const char*>(a.logits) + (long long)row * a.stride * ES;
    int a0 = (int)(((16u - (unsigned)(reinterpret_cast<uintptr_t>(rp) & 15u)) & 15u) / ES);
    if (a0 > a.V) a0 = a.V;
    const int nfull = (a.V - a0) / 8;
    const int per = (nfull + a.n_vsplit - 1) / a.n_vsplit;
    const int c0 = min(nfull, split * per), c1 = min(nfull, c0 + per);
    float m = -INFINITY, z = 0.f;
    int am = INT_MAX;
    const float c = a.c;
    if (split == 0 && threadIdx.x == 0 && a0 > 0) fold_scalar<BF16>(rp, 0, a0, m, am, z, c);
    const char* body = rp + a0 * ES;  // 16-byte aligned
    int ch = c0 + threadIdx.x;
    if (BF16) {
        for (; ch + 3 * 256 < c1; ch += 4 * 256) {
            u32x4 r[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) r[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(body + (ch + k * 256) * 16));
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                float f[8];
                unpack(r[k], f);
                fold8(f, a0 + (ch + k * 256) * 8, m, am, z, c);
            }
        }
        for (; ch < c1; ch += 256) {
            const u32x4 r = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(body + ch * 16));
            float f[8];
            unpack(r, f);
            fold8(f, a0 + ch * 8, m, am, z, c);
        }
    } else {
        for (; ch + 256 < c1; ch += 2 * 256) {
            u32x4 r[4];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                r[2 * k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(body + (ch + k * 256) * 32));
                r[2 * k + 1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(body + (ch + k * 256) * 32 + 16));
            }
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                float f[8];
                for (int e = 0; e < 4; ++e) { f[e] = __uint_as_float(r[2 * k][e]); f[4 + e] = __uint_as_float(r[2 * k + 1][e]); }
                fold8(f, a0 + (ch + k * 256) * 8, m, am, z, c);
            }
        }
        for (; ch < c1; ch += 256) {
            const u32x4 r0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(body + ch * 32));
            const u32x4 r1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(body + ch * 32 + 16));
            float f[8];
            for (int e = 0; e < 4; ++e) { f[e] = __uint_as_float(r0[e]); f[4 + e] = __uint_as_float(r1[e]); }
            fold8(f, a0 + ch * 8, m, am, z, c);
        }
    }
    const int t0 = a0 + nfull * 8;
    if (split == a.n_vsplit - 1 && threadIdx.x == 0 && t0 < a.V) fold_scalar<BF16>(rp, t0, a.V, m, am, z, c);
    // block reduction: wavefront shuffles, then across the 4 wavefronts
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float m2 = __shfl_xor(m, off);
        const int a2 = __shfl_xor(am, off);
        const float z2 = __shfl_xor(z, off);
        combine(m, am, z, m2, a2, z2, c);
    }
    __shared__ Triple sh[4];
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) sh[w] = Triple{m, am, z, 0.f};
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int k = 1; k < 4; ++k) combine(m, am, z, sh[k].m, sh[k].a, sh[k].z, c);
        a.part[(long long)split * a.B * a.S + row] = Triple{m, am, z, 0.f};
    }
}

// The 8 logits of 16-byte-aligned chunk ch of a row body, widened to float.
template <bool BF16>
__device__ __forceinline__ void load_chunk(const char* body, int ch, float (&f)[8]) {
    if (BF16) {
        unpack(*reinterpret_cast<const u32x4*>(body + (long long)ch * 16), f);
    } else {
        const u32x4 r0 = *reinterpret_cast<const u32x4*>(body + (long long)ch * 32);
        const u32x4 r1 = *reinterpret_cast<const u32x4*>(body + (long long)ch * 32 + 16);
        for (int e = 0; e < 4; ++e) { f[e] = __uint_as_float(r0[e]); f[4 + e] = __uint_as_float(r1[e]); }
    }
}

// One thread's run of a split, in increasing index order: elements [0, head)
// of the row, chunks [q0, q1) of the body (element a0 + 8 * chunk onwards),
// then elements [tail0, tail1). Adds e_v = 2^(x_v c - m c) to s one element at a
// time. With FIND it stops at the first element where base + s > r and returns
// its index (e_hit = its e_v); it returns -1 otherwise. lastpos is the last
// index seen with e_v > 0. Both instantiations perform the same additions in
// the same order, so a run that passes r in the scan also passes it here.
template <bool BF16, bool FIND>
__device__ __forceinline__ int walk_run(const char* rp, const char* body, int a0, int head, int q0, int q1,
                                        int tail0, int tail1, float c, float mc, float base, float r, float& s,
                                        int& lastpos, float& e_hit) {
    for (int v = 0; v < head; ++v) {
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(elem<BF16>(rp, v), c, -mc));
        s += e;
        if (e > 0.f) lastpos = v;
        if (FIND && base + s > r) { e_hit = e; return v; }
    }
    // chunks in batches of NB loads in flight; the additions stay in index order in both modes
    constexpr int NB = BF16 ? 16 : 8;
    int ch = q0;
    for (; ch + NB - 1 < q1; ch += NB) {
        float f[NB][8];
#pragma unroll
        for (int k = 0; k < NB; ++k) load_chunk<BF16>(body, ch + k, f[k]);
#pragma unroll
        for (int k = 0; k < NB; ++k)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(f[k][j], c, -mc));
                s += e;
                if (e > 0.f) lastpos = a0 + (ch + k) * 8 + j;
                if (FIND && base + s > r) { e_hit = e; return a0 + (ch + k) * 8 + j; }
            }
    }
    for (; ch < q1; ++ch) {
        float f[8];
        load_chunk<BF16>(body, ch, f);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(f[j], c, -mc));
            s += e;
            if (e > 0.f) lastpos = a0 + ch * 8 + j;
            if (FIND && base + s > r) { e_hit = e; return a0 + ch * 8 + j; }
        }
    }
    for (int v = tail0; v < tail1; ++v) {
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(elem<BF16>(rp, v), c, -mc));
        s += e;
        if (e > 0.f) lastpos = v;
        if (FIND && base + s > r) { e_hit = e; return v; }
    }
    return -1;
}

// Inverse transform draw for every masked row (one workgroup of 256 threads
// per row), after vocab_reduce has written the split triples.
template <bool BF16>
__global__ __launch_bounds__(256) void sample_locate(UArgs a) {
    const int row = blockIdx.x;
    if (!a.mask_in[row]) return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const long long rows = (long long)a.B * a.S;
    const float c = a.c;
    __shared__ float sh_m, sh_z, sh_r, sh_u;
    __shared__ int sh_k, sh_am;
    __shared__ float wsum[4];
    __shared__ int wfirst[4], wlast[4];
    __shared__ Triple tri[64];  // n_vsplit <= 64
    // the split triples and the uniform arrive together, one load per thread
    if (tid < a.n_vsplit) tri[tid] = a.part[(long long)tid * rows + row];
    if (tid == 128) sh_u = a.uniforms[row];
    __syncthreads();
    if (tid == 0) {
        float m = -INFINITY, z = 0.f;
        int am = INT_MAX;
        for (int k = 0; k < a.n_vsplit; ++k) combine(m, am, z, tri[k].m, tri[k].a, tri[k].z, c);
        float u = sh_u;
        u = u > 0.f ? fminf(u, 1.f) : 0.f;  // NaN and negatives count as 0
        const float t = u * z;
        int kk = -1, klast = -1;
        float W = 0.f, r = INFINITY;
        if (m != -INFINITY) {
            for (int k = 0; k < a.n_vsplit; ++k) {
                const Triple tr = tri[k];
                const float wk = tr.m == -INFINITY ? 0.f : tr.z * __builtin_amdgcn_exp2f((tr.m - m) * c);
                if (wk > 0.f) klast = k;
                if (kk < 0 && W + wk > t) { kk = k; r = t - W; }
                W += wk;
            }
            if (kk < 0) kk = klast;
        }
        sh_m = m; sh_z = z; sh_r = r; sh_k = kk; sh_am = am;
    }
    __syncthreads();
    const int k = sh_k;
    if (k < 0) {  // no logit of nonzero weight: the greedy result stands
        if (tid == 0) a.drawn[row] = Drawn{sh_am, 1.f / sh_z};
        return;
    }
    const float m = sh_m, z = sh_z, r = sh_r, mc = m * c;
    // the split's extent, cut exactly as in vocab_reduce
    constexpr int ES = BF16 ? 2 : 4;
    const char* rp = static_cast<const char*>(a.logits) + (long long)row * a.stride * ES;
    int a0 = (int)(((16u - (unsigned)(reinterpret_cast<uintptr_t>(rp) & 15u)) & 15u) / ES);
    if (a0 > a.V) a0 = a.V;
    const int nfull = (a.V - a0) / 8;
    const int per = (nfull + a.n_vsplit - 1) / a.n_vsplit;
    const int c0 = min(nfull, k * per), c1 = min(nfull, c0 + per);
    const int q = (c1 - c0 + 255) / 256;
    const int q0 = min(c1, c0 + tid * q), q1 = min(c1, q0 + q);
    const int head = (k == 0 && tid == 0) ? a0 : 0;
    const int tail0 = a0 + nfull * 8;
    const int tail1 = (k == a.n_vsplit - 1 && tid == 255) ? a.V : tail0;
    const char* body = rp + a0 * ES;
    float s = 0.f, e_hit = 0.f;
    int lastpos = -1;
    walk_run<BF16, false>(rp, body, a0, head, q0, q1, tail0, tail1, c, mc, 0.f, 0.f, s, lastpos, e_hit);
    // workgroup exclusive scan of the run sums, in thread order
    float incl = s;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
    }
    float excl = __shfl_up(incl, 1);
    if (lane == 0) excl = 0.f;
    int lp = lastpos;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) lp = max(lp, __shfl_xor(lp, off));
    if (lane == 63) wsum[w] = incl;
    if (lane == 0) wlast[w] = lp;
    __syncthreads();
    float wb = 0.f;
    for (int j = 0; j < w; ++j) wb += wsum[j];
    const float base = wb + excl;
    const unsigned long long hit = __ballot(base + s > r);
    if (lane == 0) wfirst[w] = hit ? w * 64 + __builtin_ctzll(hit) : INT_MAX;
    __syncthreads();
    const int first = min(min(wfirst[0], wfirst[1]), min(wfirst[2], wfirst[3]));
    if (first == INT_MAX) {
        // u * Z not passed inside the split (u = 1, or rounding): its last element of nonzero weight
        if (tid == 0) {
            const int last = max(max(wlast[0], wlast[1]), max(wlast[2], wlast[3]));
            if (last < 0) {
                a.drawn[row] = Drawn{sh_am, 1.f / z};
            } else {
                const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(elem<BF16>(rp, last), c, -mc));
                a.drawn[row] = Drawn{last, e / z};
            }
        }
    } else if (tid == first) {
        float s2 = 0.f;
        int lp2 = -1;
        const int v = walk_run<BF16, true>(rp, body, a0, head, q0, q1, tail0, tail1, c, mc, base, r, s2, lp2, e_hit);
        a.drawn[row] = v >= 0 ? Drawn{v, e_hit / z} : Drawn{sh_am, 1.f / z};
    }
}

__global__ __launch_bounds__(64) void unmask_select(UArgs a) {
    const int b = blockIdx.x;
    const int l = threadIdx.x;
    const bool inb = l < a.S;
    const long long row = (long long)b * a.S + l;
    const bool masked = inb && a.mask_in[row] != 0;
    float m = -INFINITY, z = 0.f;
    int am = INT_MAX;
    if (masked) {
        for (int k = 0; k < a.n_vsplit; ++k) {
            const Triple t = a.part[(long long)k * a.B * a.S + row];
            combine(m, am, z, t.m, t.a, t.z, a.c);
        }
    }
    float conf = masked ? 1.f / z : -INFINITY;
    if (masked && a.drawn) {
        const Drawn d = a.drawn[row];
        am = d.a;
        conf = d.conf;
    }
    const unsigned long long mmask = __ballot(masked);
    const int M = __popcll(mmask);
    const int kmin = (M + a.steps_left - 1) / a.steps_left;
    const bool pass = masked && conf > a.gamma;
    const int npass = __popcll(__ballot(pass));
    bool commit;
    if (npass >= kmin) {
        commit = pass;
    } else {
        int rank = 0;
        for (int j = 0; j < 64; ++j) {
            const float cj = __shfl(conf, j);
            const bool mj = (mmask >> j) & 1ull;
            if (mj && (cj > conf || (cj == conf && j < l))) ++rank;
        }
        commit = masked && rank < kmin;
    }
    const int ncommit = __popcll(__ballot(commit));
    if (inb) {
        const uint8_t old = a.mask_in[row];
        if (commit) a.tokens[row] = am;
        a.mask_out[row] = commit ? 0 : old;
        if (masked && a.conf) a.conf[row] = conf;
    }
    if (l == 0 && a.num_masked) a.num_masked[b] = M - ncommit;
}

// L_MD (section 2.2, Eq. (4)) from the (max, argmax, sum) triples of
// vocab_reduce at temperature 1: one workgroup, a thread per row, in row
// order; the loss sums in double, so it does not depend on the launch.
template <bool BF16>
__global__ __launch_bounds__(256) void nll_finish(UArgs a, const int* __restrict__ targets, float* nll, float* loss,
                                                  int* count) {
    const long long rows = (long long)a.B * a.S;
    double sum = 0.0;
    int n = 0;
    for (long long row = threadIdx.x; row < rows; row += blockDim.x) {
        if (!a.mask_in[row]) continue;
        float m = -INFINITY, z = 0.f;
        int am = INT_MAX;
        for (int k = 0; k < a.n_vsplit; ++k) {
            const Triple t = a.part[(long long)k * rows + row];
            combine(m, am, z, t.m, t.a, t.z, a.c);
        }
        const int y = targets[row];
        float v = __builtin_nanf("");
        if (y >= 0 && y < a.V) {
            const char* rp = static_cast<const char*>(a.logits) + row * a.stride * (BF16 ? 2 : 4);
            v = m + __logf(z) - elem<BF16>(rp, y);
        }
        if (nll) nll[row] = v;
        sum += (double)v;
        ++n;
    }
    __shared__ double ss[256];
    __shared__ int sn[256];
    ss[threadIdx.x] = sum;
    sn[threadIdx.x] = n;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
        if ((int)threadIdx.x < off) {
            ss[threadIdx.x] += ss[threadIdx.x + off];
            sn[threadIdx.x] += sn[threadIdx.x + off];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        *loss = sn[0] > 0 ? (float)(ss[0] / sn[0]) : 0.f;
        if (count) *count = sn[0];
    }
}

}  // namespace

UnmaskPlan plan_unmask(const tt_conf_unmask_params& p, int n_cu) {
    UnmaskPlan pl{};
    const long long rows = (long long)p.B * p.S;
    const int cu = n_cu > 0 ? n_cu : 256;
    // enough workgroups to cover the chip about 8 times, at least 2048 logits each
    long long want = rows > 0 ? (8LL * cu + rows - 1) / rows : 1;
    long long cap = (p.V + 2047) / 2048;
    if (want > cap) want = cap;
    if (want < 1) want = 1;
    if (want > 64) want = 64;
    pl.n_vsplit = (int)want;
    pl.ws_part = (size_t)pl.n_vsplit * (size_t)rows * sizeof(Triple);
    pl.ws_total = pl.ws_part + (p.uniforms ? (size_t)rows * sizeof(Drawn) : 0);
    return pl;
}

tt_status launch_unmask(const tt_conf_unmask_params& p, const UnmaskPlan& pl, void* ws, hipStream_t s) {
    UArgs a{};
    a.logits = p.logits;
    a.stride = p.logits_stride_row;
    a.mask_in = p.mask_in;
    a.mask_out = p.mask_out;
    a.tokens = p.tokens;
    a.conf = p.conf;
    a.num_masked = p.num_masked;
    a.part = static_cast<Triple*>(ws);
    a.B = p.B; a.S = p.S; a.V = p.V;
    a.n_vsplit = pl.n_vsplit;
    a.steps_left = p.steps_left;
    a.gamma = p.gamma;
    a.c = 1.44269504088896340736f / p.temperature;
    a.uniforms = p.uniforms;
    a.drawn = p.uniforms ? reinterpret_cast<Drawn*>(static_cast<char*>(ws) + pl.ws_part) : nullptr;
    const dim3 grid(p.B * p.S, pl.n_vsplit);
    if (p.dtype == TT_BF16)
        hipLaunchKernelGGL(vocab_reduce<true>, grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(vocab_reduce<false>, grid, dim3(256), 0, s, a);
    if (p.uniforms) {
        if (p.dtype == TT_BF16)
            hipLaunchKernelGGL(sample_locate<true>, dim3(p.B * p.S), dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL(sample_locate<false>, dim3(p.B * p.S), dim3(256), 0, s, a);
    }
    hipLaunchKernelGGL(unmask_select, dim3(p.B), dim3(64), 0, s, a);
    return hipGetLastError() == hipSuccess ? TT_OK : TT_ERR_HIP;
}

UnmaskPlan plan_nll(const tt_masked_nll_params& p, int n_cu) {
    tt_conf_unmask_params u{};
    u.B = p.B;
    u.S = p.S;
    u.V = p.V;
    return plan_unmask(u, n_cu);
}

tt_status launch_nll(const tt_masked_nll_params& p, const UnmaskPlan& pl, void* ws, hipStream_t s) {
    UArgs a{};
    a.logits = p.logits;
    a.stride = p.logits_stride_row;
    a.mask_in = p.mask;
    a.part = static_cast<Triple*>(ws);
    a.B = p.B; a.S = p.S; a.V = p.V;
    a.n_vsplit = pl.n_vsplit;
    a.c = 1.44269504088896340736f;  // temperature 1
    const dim3 grid(p.B * p.S, pl.n_vsplit);
    if (p.dtype == TT_BF16) {
        hipLaunchKernelGGL(vocab_reduce<true>, grid, dim3(256), 0, s, a);
        hipLaunchKernelGGL(nll_finish<true>, dim3(1), dim3(256), 0, s, a, p.targets, p.nll, p.loss, p.count);
    } else {
        hipLaunchKernelGGL(vocab_reduce<false>, grid, dim3(256), 0, s, a);
        hipLaunchKernelGGL(nll_finish<false>, dim3(1), dim3(256), 0, s, a, p.targets, p.nll, p.loss, p.count);
    }
    return hipGetLastError() == hipSuccess ? TT_OK : TT_ERR_HIP;
}

}  // namespace tt
