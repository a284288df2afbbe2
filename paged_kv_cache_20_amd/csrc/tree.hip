// tree.hip -- a speculative round shaped as a tree ("Radiance Architecture
// Plugins -- declaring a model", section "Declare: drafters, encoders,
// generators": a drafter may propose a tree; "TandemLLM -- Adding a model",
// section "The adapter path in ten steps": a recorded decode replayed as
// trees of every verify width must match row for row, bit for bit).
//
// Row r of a round of R rows sits in the cache at position C0 + r
// (C0 = ctx_len - R) and attends the cached context 0 .. C0 - 1 plus the
// round rows its mask names (its ancestors and itself, in row order).  Its
// result is, bit for bit, the decode of that branch: the branch's tokens laid
// at positions C0, C0 + 1, ... of an otherwise identical cache.
//
// This file builds, for every (sequence, row), that branch view: a private
// copy of the page holding C0 (its context rows and the branch tokens that
// land in it) and of the next page if the branch spills into it, written to
// two caller-reserved pool pages, a block-table row that is the sequence's
// own up to the page before C0 and the private pages after, the view's length
// and the first key of the split holding C0.  The decode kernels then
// run over the views (the splits below C0's on the sequence's own pages for
// all rows at once, C0's split and the next per view, then one combine per
// view), so a row's arithmetic is exactly the decode's.  bf16 bytes are
// copied.  An fp8 view page takes the scale of the cache page holding its
// first token and copies that page's codes; where a round crosses a page
// boundary and the branch skips rows, later rows move down into the earlier
// page, and those are written as an append into that page at a later call
// would write them: each moved value (code times its own page's scale, fp32)
// is encoded at the view page's scale, which first doubles while the moved
// values do not fit (448 times the scale), re-encoding the page's other codes
// at the grown scale.  A chain mask moves nothing, so its views are the cache.
// A row whose view cannot be formed (bad mask, bad page) gets length 0 and so
// NaN.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "e4m3.h"
#include "kernels.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One workgroup per (sequence, row).  Thread layout: 16-byte pieces of the
// rows to copy, (row of the view page, kv head, piece) flattened.
__global__ __launch_bounds__(256) void tree_stage_kernel(TreeArgs a)
{
    const int sr = blockIdx.x;  // s * R + r
    const int R = a.rows;
    const int s = sr / R, r = sr - s * R;
    const int C = a.ctx_lens[s];
    const int Hk = a.n_head_kv;
    const int eb = a.fp8 ? 1 : 2;
    const int rowb = a.head_dim * eb;  // bytes of one token row of one kv head
    const int pieces = rowb / 16;
    const int64_t chunkb = (int64_t)16 * rowb;  // one (page, kv head)
    const int64_t pageb = chunkb * Hk;
    int32_t* vt = a.vtable + (int64_t)sr * a.max_pages;

    const int C0 = C - R;
    const uint32_t mask = (uint32_t)a.tree_mask[(int64_t)s * R + r];
    // Valid view: sane length, the row names itself and no later row.
    bool ok = C >= R && (int64_t)C <= (int64_t)a.max_pages * 16 &&
              (mask >> r & 1u) != 0 && (mask >> (r + 1)) == 0;
    const int depth = __builtin_popcount(mask);
    const int L = C0 + depth;        // length of the branch view
    const int tp = C0 >> 4;          // page holding C0
    const int npriv = ((L - 1) >> 4) - tp + 1;  // private pages (1 or 2)
    int32_t priv[2];
    for (int i = 0; i < 2; ++i) {
        priv[i] = a.scratch[(int64_t)sr * 2 + i];
        if (i < npriv && (priv[i] < 0 || (int64_t)priv[i] >= a.n_pages))
            ok = false;
    }
    // Source pages: the sequence's pages tp and tp + 1 (round rows live there).
    int32_t src[2];
    for (int i = 0; i < 2; ++i) {
        const int e = tp + i;
        src[i] = (ok && e * 16 < C) ? a.block_table[(int64_t)s * a.max_pages + e] : 0;
        if (ok && e * 16 < C && (src[i] < 0 || (int64_t)src[i] >= a.n_pages))
            ok = false;
    }

    // The view's table row and length.
    for (int e = threadIdx.x; e < a.max_pages; e += blockDim.x) {
        int32_t v = -1;
        if (ok) {
            if (e < tp)
                v = a.block_table[(int64_t)s * a.max_pages + e];
            else if (e - tp < npriv)
                v = priv[e - tp];
        }
        vt[e] = v;
    }
    if (threadIdx.x == 0) {
        a.vlens[sr] = ok ? L : 0;
        a.vfloor[sr] = ok ? (C0 / a.chunk) * a.chunk : 0;
    }
    if (!ok)
        return;

    // Position of view row v (C0 .. L-1) in the cache: the i-th named round row.
    auto branch_pos = [&](int i) {
        uint32_t m = mask;
        for (int k = 0; k < i; ++k)
            m &= m - 1;  // drop the lowest set bit i times
        return C0 + __builtin_ctz(m);
    };
    // Rows of the private pages: [tp*16, L).  Context rows below C0 come from
    // page src[0]; view rows from their branch tokens.  With fp8 the rows of
    // the first private page are written by the pass below.
    const int first = tp * 16;
    const int t_hi = L < first + 16 ? L : first + 16;  // end of the first private page
    const int cfirst = a.fp8 ? t_hi : first;
    const int64_t total = (int64_t)(L - cfirst) * Hk * pieces;
    uint8_t* kp = (uint8_t*)a.k_pool;
    uint8_t* vp = (uint8_t*)a.v_pool;
    for (int64_t t = threadIdx.x; t < total; t += blockDim.x) {
        const int piece = (int)(t % pieces);
        const int64_t rest = t / pieces;
        const int kh = (int)(rest % Hk);
        const int vrow = cfirst + (int)(rest / Hk);  // view position
        const int pos = vrow < C0 ? vrow : branch_pos(vrow - C0);
        const int32_t sp = src[(pos >> 4) - tp];
        const int32_t dp = priv[(vrow >> 4) - tp];
        const int64_t so = sp * pageb + kh * chunkb + (int64_t)(pos & 15) * rowb + piece * 16;
        const int64_t dofs = dp * pageb + kh * chunkb + (int64_t)(vrow & 15) * rowb + piece * 16;
        *(u32x4*)(kp + dofs) = *(const u32x4*)(kp + so);
        *(u32x4*)(vp + dofs) = *(const u32x4*)(vp + so);
    }
    if (!a.fp8)
        return;
    // fp8, first private page: one wave per (kv head, K or V).  Rows from
    // page src[0] keep their codes unless the scale grows; rows from src[1]
    // (moved down) are re-encoded.  The second private page, if any, holds
    // rows of src[1] only and takes its scale.
    const int lane = threadIdx.x & 63;
    const bool has_next = (tp + 1) * 16 < C;
    for (int pair = threadIdx.x >> 6; pair < 2 * Hk; pair += blockDim.x >> 6) {
        const int kv = pair & 1, kh = pair >> 1;
        uint8_t* pool = kv ? vp : kp;
        float* scales = kv ? a.v_scale : a.k_scale;
        const float s_home = scales[(int64_t)src[0] * Hk + kh];
        const float s_next = has_next ? scales[(int64_t)src[1] * Hk + kh] : 1.f;
        float amax = 0.f;
        for (int v = C0; v < t_hi; ++v) {
            const int pos = branch_pos(v - C0);
            if ((pos >> 4) == tp)
                continue;
            const uint8_t* row = pool + src[1] * pageb + kh * chunkb + (int64_t)(pos & 15) * rowb;
            for (int i = lane; i < a.head_dim; i += 64)
                amax = __builtin_fmaxf(amax, __builtin_fabsf(e4m3_value(row[i]) * s_next));
        }
#pragma unroll
        for (int msk = 32; msk >= 1; msk >>= 1)
            amax = __builtin_fmaxf(amax, __shfl_xor(amax, msk, 64));
        float s_view = s_home;
        if (amax <= 3.4028234663852886e38f && amax / s_home > 448.f)
            while (amax / s_view > 448.f)
                s_view = s_view * 2.f;
        const bool grown = s_view != s_home;
        for (int v = first; v < t_hi; ++v) {
            const int pos = v < C0 ? v : branch_pos(v - C0);
            const int moved = (pos >> 4) != tp;
            const float s = moved ? s_next : s_home;
            const uint8_t* srow = pool + src[moved] * pageb + kh * chunkb + (int64_t)(pos & 15) * rowb;
            uint8_t* drow = pool + priv[0] * pageb + kh * chunkb + (int64_t)(v & 15) * rowb;
            for (int i = lane; i < a.head_dim; i += 64) {
                uint32_t c = srow[i];
                if (moved || grown)
                    c = e4m3_code(e4m3_value(c) * s / s_view);
                drow[i] = (uint8_t)c;
            }
        }
        if (lane == 0) {
            scales[(int64_t)priv[0] * Hk + kh] = s_view;
            if (npriv == 2)
                scales[(int64_t)priv[1] * Hk + kh] = s_next;
        }
    }
}

}  // namespace

hipError_t launch_tree_stage(const TreeArgs& a, hipStream_t stream)
{
    hipLaunchKernelGGL(tree_stage_kernel, dim3((unsigned)(a.n_seq * a.rows)), dim3(256), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace pa
