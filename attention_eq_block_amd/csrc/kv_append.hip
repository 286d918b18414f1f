// Commit-time KV append (Nemotron-TwoTower, arXiv 2606.26493, section 2.1,
// Algorithm 1: after a block is committed the context tower extends its
// per-layer KV cache, so the next block attends to a prefix longer by S).
//
// Two launches on the caller's stream:
//   kv_append_plan  one wave: checks every sequence (capacity, page ids, pool
//                   size), then gives each needed page-table entry a page from
//                   the top of the pool in (sequence, position) order, grows
//                   ctx_len by S and writes the status. It changes nothing
//                   when a check fails.
//   kv_append_copy  one workgroup per new row (b, s): 16-byte copies of the
//                   row's K and V for every KV head into the slot the table
//                   now names. It does nothing when the plan failed.
// The copy is HBM-bound and tiny next to the attention it feeds (about 1 MB
// per layer for a batch of 32 blocks of 16 tokens).
#include "tt_internal.h"

namespace tt {
namespace {

struct AppendArgs {
    int B, S, Hkv, row_bytes;  // row_bytes: head_dim * element size (multiple of 16)
    int page_size, num_pages, max_pages;
    char* Kc;
    char* Vc;
    int* table;
    int* ctx_len;
    const char* Kn;
    const char* Vn;
    long long nsb, nss, nsh;  // byte strides of the new rows
    const int* pool;
    int* pool_count;
    int* status;
};

// x of another lane by a DPP pattern (0 where the pattern names none or the
// row is masked off): a register move, no LDS round trip
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_move(int x) {
    return __builtin_amdgcn_update_dpp(0, x, CTRL, ROWS, 0xF, false);
}

// Inclusive prefix sum over the 64 lanes of a wave (all active): within each row
// of 16 lanes by shifts of 1, 2, 4 and 8, then row 0's total into row 1 and row
// 2's into row 3 (broadcast of lanes 15 and 47), then that of rows 0-1 into rows
// 2 and 3 (broadcast of lane 31)
__device__ __forceinline__ int wave_incl_sum(int x, int) {
    x += dpp_move<0x111, 0xF>(x);  // row_shr:1
    x += dpp_move<0x112, 0xF>(x);  // row_shr:2
    x += dpp_move<0x114, 0xF>(x);  // row_shr:4
    x += dpp_move<0x118, 0xF>(x);  // row_shr:8
    x += dpp_move<0x142, 0xA>(x);  // row_bcast:15, rows 1 and 3
    x += dpp_move<0x143, 0xC>(x);  // row_bcast:31, rows 2 and 3
    return x;
}

// pages of [first, last] of sequence b that have no page yet; flags a page id
// outside [0, num_pages) in `bad`
__device__ __forceinline__ int pages_needed(const AppendArgs& a, int b, int L, bool& bad) {
    const int p0 = L / a.page_size, p1 = (L + a.S - 1) / a.page_size;
    int need = 0;
    for (int p = p0; p <= p1; ++p) {
        const int e = a.table[(long long)b * a.max_pages + p];
        if (e < 0) ++need;
        else if (e >= a.num_pages) bad = true;
    }
    return need;
}

__global__ __launch_bounds__(64) void kv_append_plan(AppendArgs a) {
    const int lane = threadIdx.x;
    const long long cap = (long long)a.max_pages * a.page_size;
    const int count = a.pool_count ? max(*a.pool_count, 0) : 0;
    // checks
    bool cap_bad = false, page_bad = false;
    int total = 0;
    for (int base = 0; base < a.B; base += 64) {
        const int b = base + lane;
        int need = 0;
        if (b < a.B) {
            const int L = max(a.ctx_len[b], 0);
            if ((long long)L + a.S > cap) cap_bad = true;
            else need = pages_needed(a, b, L, page_bad);
        }
        total += __builtin_amdgcn_readlane(wave_incl_sum(need, lane), 63);
    }
    const bool any_cap = __builtin_amdgcn_ballot_w64(cap_bad) != 0;
    if (!any_cap && total <= count) {
        for (int k = lane; k < total; k += 64) {
            const int pg = a.pool[count - 1 - k];
            if (pg < 0 || pg >= a.num_pages) page_bad = true;
        }
    }
    const bool any_page = __builtin_amdgcn_ballot_w64(page_bad) != 0;
    const int code = any_cap ? 1 : (total > count ? 2 : (any_page ? 3 : 0));
    if (code != 0) {
        if (lane == 0) *a.status = code;
        return;
    }
    // assignment: the k-th page needed overall takes pool[count - 1 - k]
    int carry = 0;
    for (int base = 0; base < a.B; base += 64) {
        const int b = base + lane;
        int need = 0, L = 0;
        bool unused = false;
        if (b < a.B) {
            L = max(a.ctx_len[b], 0);
            need = pages_needed(a, b, L, unused);
        }
        const int incl = wave_incl_sum(need, lane);
        int k = carry + incl - need;
        if (b < a.B) {
            const int p0 = L / a.page_size, p1 = (L + a.S - 1) / a.page_size;
            for (int p = p0; p <= p1; ++p) {
                int* e = a.table + (long long)b * a.max_pages + p;
                if (*e < 0) *e = a.pool[count - 1 - k++];
            }
            a.ctx_len[b] = L + a.S;
        }
        carry += __builtin_amdgcn_readlane(incl, 63);
    }
    if (lane == 0) {
        if (total > 0) *a.pool_count = count - total;
        *a.status = 0;
    }
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(64) void kv_append_copy(AppendArgs a) {
    if (*a.status != 0) return;
    const int b = blockIdx.x / a.S, s = blockIdx.x % a.S;
    const int j = a.ctx_len[b] - a.S + s;  // ctx_len already grown by the plan
    const int page = a.table[(long long)b * a.max_pages + j / a.page_size];
    const int slot = j % a.page_size;
    const int chunks = a.row_bytes / 16;  // per KV head
    const int n = 2 * a.Hkv * chunks;
    for (int c = threadIdx.x; c < n; c += blockDim.x) {
        const int kv = c / (a.Hkv * chunks);
        const int g = (c / chunks) % a.Hkv, w = c % chunks;
        const char* src = (kv ? a.Vn : a.Kn) + b * a.nsb + s * a.nss + g * a.nsh + w * 16;
        char* dst = (kv ? a.Vc : a.Kc) + (((long long)page * a.Hkv + g) * a.page_size + slot) * a.row_bytes + w * 16;
        *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
    }
}

}  // namespace

tt_status launch_kv_append(const tt_kv_append_params& p, hipStream_t s) {
    AppendArgs a{};
    const int esz = p.dtype == TT_BF16 ? 2 : 4;
    a.B = p.B; a.S = p.S; a.Hkv = p.Hkv; a.row_bytes = p.head_dim * esz;
    a.page_size = p.page_size; a.num_pages = p.num_pages; a.max_pages = p.max_pages;
    a.Kc = static_cast<char*>(p.Kctx);
    a.Vc = static_cast<char*>(p.Vctx);
    a.table = p.page_table;
    a.ctx_len = p.ctx_len;
    a.Kn = static_cast<const char*>(p.Knew);
    a.Vn = static_cast<const char*>(p.Vnew);
    a.nsb = p.new_stride_b * esz; a.nss = p.new_stride_s * esz; a.nsh = p.new_stride_h * esz;
    a.pool = p.pool;
    a.pool_count = p.pool_count;
    a.status = p.status;
    hipLaunchKernelGGL(kv_append_plan, dim3(1), dim3(64), 0, s, a);
    hipLaunchKernelGGL(kv_append_copy, dim3(p.B * p.S), dim3(64), 0, s, a);
    return hipGetLastError() == hipSuccess ? TT_OK : TT_ERR_HIP;
}

}  // namespace tt
