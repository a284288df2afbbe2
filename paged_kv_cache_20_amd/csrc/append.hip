// append.hip -- write a call's new K/V rows into their paged token slots
// ("kern manifest v7" schema, $defs.Fill "slot": each row's token slot in
// the paged state; slot = page * 16 + offset), quantising to e4m3 for fp8
// caches.
//
// fp8: one scale per (page, kv head), separately for K and V, set to
// absmax / 448 by the call that writes the page's offset 0, over that call's
// rows in the page (the "one fp32 scale per page per KV head (absmax/448)"
// layout).  A later call keeps the stored scale while its rows fit (fp32
// absmax / scale <= 448); otherwise it doubles the scale until they fit and
// re-encodes the codes already in the page's earlier slots at the new scale
// (exact for every code that stays a normal number), so rows appended one
// token at a time keep E4M3's precision.  A code is the OCP E4M3 value
// nearest to x / scale (fp32 quotient), ties to even, saturating at 448.
// The rows a call writes into one page must be one run of consecutive rows
// at consecutive offsets: runs of one page are not ordered against each
// other.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "e4m3.h"
#include "kernels.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// bf16: one thread per 16-byte piece of a K (and the same V) row.
template <int D>
__global__ __launch_bounds__(256) void append_bf16(AppendArgs a)
{
    constexpr int PPR = D / 8;  // pieces per (token, head)
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t per_tok = (int64_t)a.n_head_kv * PPR;
    if (idx >= (int64_t)a.n_tok * per_tok)
        return;
    const int64_t t = idx / per_tok;
    const int c = (int)(idx - t * per_tok);
    const int h = c / PPR, e = c - h * PPR;
    const int64_t slot = a.slots[t];
    if (slot < 0 || slot >= a.n_pages * 16)
        return;
    const int64_t page = slot >> 4, off = slot & 15;
    const int64_t dst = ((page * a.n_head_kv + h) * 16 + off) * D + e * 8;
    const int64_t src = (t * a.n_head_kv + h) * D + e * 8;
    *(u32x4*)((uint16_t*)a.k_pool + dst) = *(const u32x4*)((const uint16_t*)a.k_new + src);
    *(u32x4*)((uint16_t*)a.v_pool + dst) = *(const u32x4*)((const uint16_t*)a.v_new + src);
}

// fp8: one wave per (row, kv head) that starts a run of rows landing in one
// page at consecutive offsets; the wave sets the scales (if the run starts at
// offset 0), grows them (re-encoding the page's earlier codes) if the run
// does not fit, and writes the run's codes.
template <int D>
__global__ __launch_bounds__(256) void append_fp8(AppendArgs a)
{
    constexpr int E = D / 64;  // elements per lane per row
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int h = blockIdx.y;
    if (t >= a.n_tok)
        return;
    const int64_t cap = a.n_pages * 16;
    const int64_t slot = a.slots[t];
    if (slot < 0 || slot >= cap)
        return;
    if (t > 0) {
        const int64_t prev = a.slots[t - 1];
        if (prev >= 0 && prev < cap && prev == slot - 1 && (prev >> 4) == (slot >> 4))
            return;  // not the first row of its run
    }
    const int64_t page = slot >> 4;
    const int off = (int)(slot & 15);
    int len = 1;
    while (off + len < 16 && t + len < a.n_tok && (int64_t)a.slots[t + len] == slot + len)
        ++len;

    const int Hk = a.n_head_kv;
    const int64_t sc_idx = page * Hk + h;
    for (int kv = 0; kv < 2; ++kv) {
        const uint16_t* src = (const uint16_t*)(kv ? a.v_new : a.k_new);
        uint8_t* pool = (uint8_t*)(kv ? a.v_pool : a.k_pool);
        float* scales = kv ? a.v_scale : a.k_scale;
        float amax = 0.f;
        for (int u = 0; u < len; ++u) {
            const uint16_t* row = src + ((int64_t)(t + u) * Hk + h) * D;
#pragma unroll
            for (int e = 0; e < E; ++e)
                amax = __builtin_fmaxf(amax, __builtin_fabsf(bf16_to_f32(row[lane + 64 * e])));
        }
#pragma unroll
        for (int msk = 32; msk >= 1; msk >>= 1)
            amax = __builtin_fmaxf(amax, __shfl_xor(amax, msk, 64));
        float scale;
        if (off == 0) {
            scale = amax > 0.f ? amax / 448.f : 1.f;
            if (lane == 0)
                scales[sc_idx] = scale;
        } else {
            scale = scales[sc_idx];
            if (amax <= 3.4028234663852886e38f && amax / scale > 448.f) {
                float ns = scale;
                while (amax / ns > 448.f)
                    ns = ns * 2.f;
                for (int u = 0; u < off; ++u) {
                    uint8_t* row = pool + ((page * Hk + h) * 16 + u) * D;
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const float y = e4m3_value(row[lane + 64 * e]) * scale;
                        row[lane + 64 * e] = (uint8_t)e4m3_code(y / ns);
                    }
                }
                scale = ns;
                if (lane == 0)
                    scales[sc_idx] = ns;
            }
        }
        for (int u = 0; u < len; ++u) {
            const uint16_t* row = src + ((int64_t)(t + u) * Hk + h) * D;
            uint8_t* dst = pool + ((page * Hk + h) * 16 + off + u) * D;
#pragma unroll
            for (int e = 0; e < E; ++e)
                dst[lane + 64 * e] = (uint8_t)e4m3_code(bf16_to_f32(row[lane + 64 * e]) / scale);
        }
    }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t stream)
{
    if (a.n_tok <= 0)
        return hipSuccess;
    if (!a.fp8) {
        const int64_t threads = (int64_t)a.n_tok * a.n_head_kv * (a.head_dim / 8);
        const dim3 grid((unsigned)((threads + 255) / 256));
        if (a.head_dim == 128)
            hipLaunchKernelGGL(append_bf16<128>, grid, dim3(256), 0, stream, a);
        else if (a.head_dim == 256)
            hipLaunchKernelGGL(append_bf16<256>, grid, dim3(256), 0, stream, a);
        else
            return hipErrorNotSupported;
    } else {
        const dim3 grid((unsigned)((a.n_tok + 3) / 4), (unsigned)a.n_head_kv);
        if (a.head_dim == 128)
            hipLaunchKernelGGL(append_fp8<128>, grid, dim3(256), 0, stream, a);
        else if (a.head_dim == 256)
            hipLaunchKernelGGL(append_fp8<256>, grid, dim3(256), 0, stream, a);
        else
            return hipErrorNotSupported;
    }
    return hipGetLastError();
}

}  // namespace pa
