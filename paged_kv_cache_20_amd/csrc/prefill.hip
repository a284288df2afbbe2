// prefill.hip -- a chunk of new rows of ONE sequence over its paged cache
// ("kern manifest v7" schema, $defs.Batch: one sequence, as many rows as the
// chunk; `context` is the cached rows the call expands over).  Row r of an
// n_rows chunk sits at position ctx_len - n_rows + r and attends to keys
// 0 .. that position.
//
// Work decomposition (gfx950)
//   A workgroup of 4 waves owns one kv head and 128 query rows: 128/g
//   consecutive positions x the g query heads that share the kv head, so
//   every K/V tile it stages serves g heads.  Wave w owns rows 32w..32w+31.
//   Keys stream in 64-key tiles (four 16-token pages) through two LDS
//   buffers: while the waves compute on one, the next tile's K and V rows
//   are in flight from the paged pools into registers and then written to
//   the other buffer (K row-major; V transposed to [d][key] with a 4-key x
//   8-element register transpose so LDS writes are 8 bytes wide).
//   Per wave and tile, on v_mfma_f32_32x32x16_bf16:
//     S^T[key][row] = K . Q^T      Q^T lives in registers for the whole call
//     online softmax               each lane owns one row: its 32 scores of
//                                  the tile sit in the lane (plus its pair
//                                  lane 32 away), so max/sum need one swap
//     O^T[d][row]  += V^T . P^T    P^T is the S^T accumulator re-packed in
//                                  place; O^T's row is again the lane's row,
//                                  so rescaling and the final 1/l stay local
//   fp8 pages are converted to bf16 exactly on the way into LDS; the K scale
//   multiplies the scores and the V scale is folded into P, per page.
//   Workgroups of one kv head are placed on the same XCDs (blockIdx mod 8
//   picks the XCD) so the K/V tiles they stream share that XCD's L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kKT = 64;  // keys per tile

__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }

__device__ __forceinline__ uint32_t bf16_bits(float x)
{
    __bf16 b = (__bf16)x;
    return (uint32_t)__builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    return bf16_bits(lo) | (bf16_bits(hi) << 16);
}

template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w)
{
    bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HI);
    return __builtin_bit_cast(uint32_t, r);
}

template <int D, bool FP8>
struct PGeo {
    static constexpr int EB = FP8 ? 1 : 2;
    static constexpr int ROWB = D * EB;        // bytes of one token row in the pool
    static constexpr int CPR = ROWB / 16;      // 16-byte chunks per pool row
    static constexpr int EPC = 16 / EB;        // elements per chunk
    static constexpr int KCH = kKT * CPR / 256;  // K chunks per thread per tile
    static constexpr int VUN = 16 * CPR;       // V units (4 keys x 1 chunk) per tile
    static constexpr int VUT = (VUN + 255) / 256;  // V units per thread (last may idle)
    static constexpr int KS = D * 2 + 16;      // LDS K row stride (bytes)
    static constexpr int VS = kKT * 2 + 8;     // LDS V^T row stride (bytes)
    static constexpr int KBYTES = kKT * KS;
    static constexpr int VBYTES = D * VS;
    static constexpr int SBYTES = 64;          // per-page scales of the tile (fp8)
    static constexpr int BUF = KBYTES + VBYTES + SBYTES;
    static constexpr int DSTEPS = D / 16;      // k-steps of QK^T
    static constexpr int DBLK = D / 32;        // 32-wide d blocks of O^T
};

template <int D, bool FP8>
struct Stage {  // one thread's share of a tile in flight
    u32x4 k[PGeo<D, FP8>::KCH];
    u32x4 v[PGeo<D, FP8>::VUT][4];
    float ks, vs;  // threads 0..3: scales of page tid of the tile
};

struct Blk {
    int C, n_rows, base_pos, kh, Hk;
    int64_t n_pages;
    const int32_t* bt;
};

// Page id of key `key` (or -1 when the key is at or past the context).
__device__ __forceinline__ int page_of(const Blk& b, int key, int* bad)
{
    if (key >= b.C)
        return -1;
    const int p = b.bt[key >> 4];
    if (p < 0 || (int64_t)p >= b.n_pages) {
        *bad = 1;
        return -1;
    }
    return p;
}

template <int D, bool FP8>
__device__ __forceinline__ void stage_load(Stage<D, FP8>& st, const Blk& b, const uint8_t* kp,
                                           const uint8_t* vp, const float* ksc, const float* vsc,
                                           int tile0, int tid, int* bad)
{
    using G = PGeo<D, FP8>;
#pragma unroll
    for (int i = 0; i < G::KCH; ++i) {
        const int c = i * 256 + tid;
        const int key = c / G::CPR, piece = c % G::CPR;
        const int pg = page_of(b, tile0 + key, bad);
        if (pg >= 0)
            st.k[i] = *(const u32x4*)(kp + (((int64_t)pg * b.Hk + b.kh) * 16 + ((tile0 + key) & 15)) *
                                               G::ROWB + piece * 16);
        else
            st.k[i] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < G::VUT; ++i) {
        const int u = i * 256 + tid;
        const int kg = u & 15, piece = u >> 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int key = tile0 + 4 * kg + j;
            const int pg = u < G::VUN ? page_of(b, key, bad) : -1;
            if (pg >= 0)
                st.v[i][j] = *(const u32x4*)(vp + (((int64_t)pg * b.Hk + b.kh) * 16 + (key & 15)) *
                                                      G::ROWB + piece * 16);
            else
                st.v[i][j] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    if (FP8 && tid < 4) {
        const int pg = page_of(b, tile0 + 16 * tid, bad);
        st.ks = pg >= 0 ? ksc[(int64_t)pg * b.Hk + b.kh] : 0.f;
        st.vs = pg >= 0 ? vsc[(int64_t)pg * b.Hk + b.kh] : 0.f;
    }
}

template <int D, bool FP8>
__device__ __forceinline__ void stage_store(const Stage<D, FP8>& st, char* buf, int tid)
{
    using G = PGeo<D, FP8>;
    char* ks = buf;
    char* vt = buf + G::KBYTES;
    float* sc = (float*)(buf + G::KBYTES + G::VBYTES);
#pragma unroll
    for (int i = 0; i < G::KCH; ++i) {
        const int c = i * 256 + tid;
        const int key = c / G::CPR, piece = c % G::CPR;
        if constexpr (FP8) {
            const u32x4 w = st.k[i];
            u32x4 lo, hi;
            lo[0] = fp8x2_to_bf16x2<false>(w[0]);
            lo[1] = fp8x2_to_bf16x2<true>(w[0]);
            lo[2] = fp8x2_to_bf16x2<false>(w[1]);
            lo[3] = fp8x2_to_bf16x2<true>(w[1]);
            hi[0] = fp8x2_to_bf16x2<false>(w[2]);
            hi[1] = fp8x2_to_bf16x2<true>(w[2]);
            hi[2] = fp8x2_to_bf16x2<false>(w[3]);
            hi[3] = fp8x2_to_bf16x2<true>(w[3]);
            *(u32x4*)(ks + key * G::KS + piece * 32) = lo;
            *(u32x4*)(ks + key * G::KS + piece * 32 + 16) = hi;
        } else {
            *(u32x4*)(ks + key * G::KS + piece * 16) = st.k[i];
        }
    }
#pragma unroll
    for (int i = 0; i < G::VUT; ++i) {
        const int u = i * 256 + tid;
        if (u >= G::VUN)
            continue;
        const int kg = u & 15, piece = u >> 4;
        // bf16 elements of the 4 keys: dword w of key j holds elements 2w, 2w+1
        uint32_t e[4][G::EPC / 2];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (FP8) {
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    e[j][2 * w] = fp8x2_to_bf16x2<false>(st.v[i][j][w]);
                    e[j][2 * w + 1] = fp8x2_to_bf16x2<true>(st.v[i][j][w]);
                }
            } else {
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    e[j][w] = st.v[i][j][w];
            }
        }
#pragma unroll
        for (int x = 0; x < G::EPC; ++x) {
            const uint32_t sel = (x & 1) ? 0x07060302u : 0x05040100u;
            u32x2 o;
            o[0] = __builtin_amdgcn_perm(e[1][x >> 1], e[0][x >> 1], sel);
            o[1] = __builtin_amdgcn_perm(e[3][x >> 1], e[2][x >> 1], sel);
            const int d = piece * G::EPC + x;
            *(u32x2*)(vt + d * G::VS + kg * 8) = o;
        }
    }
    if (FP8 && tid < 4) {
        sc[tid] = st.ks;
        sc[4 + tid] = st.vs;
    }
}

template <int D, bool FP8>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillArgs a)
{
    using G = PGeo<D, FP8>;
    __shared__ __attribute__((aligned(16))) char smem[2 * G::BUF];
    __shared__ int s_bad;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, kb = lane >> 5;
    const int Hk = a.n_head_kv, H = a.n_head, g = H / Hk, BP = 128 / g;
    const int npb = (a.n_rows + BP - 1) / BP;
    const int nblk = npb * Hk;
    // XCD-aware placement: consecutive list entries (same kv head) go to the
    // same XCD; heavier (later) position blocks first within a kv head.
    const int per_xcd = (nblk + 7) / 8;
    const int L = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (L >= nblk)
        return;
    const int kh = L / npb;
    const int pb = npb - 1 - (L - kh * npb);

    Blk b;
    b.C = a.ctx_len;
    b.n_rows = a.n_rows;
    b.base_pos = a.ctx_len - a.n_rows;
    b.kh = kh;
    b.Hk = Hk;
    b.n_pages = a.n_pages;
    b.bt = a.block_table;

    // This lane's query row.
    const int wrow = 32 * wave + l32;          // 0..127 in the workgroup
    const int hg = wrow / BP, p = wrow - hg * BP;
    const int r = pb * BP + p;                 // row of the call
    const bool valid = r < a.n_rows;
    const int h = kh * g + hg;
    const int pos = valid ? b.base_pos + r : -1;
    const int rlast = min(a.n_rows, (pb + 1) * BP) - 1;
    const int maxpos = b.base_pos + rlast;     // last key any row here needs
    const int minpos = b.base_pos + pb * BP;
    const int nt = (maxpos + kKT) / kKT;

    // Q^T operand: 8 bf16 of row `wrow` per k-step (d = 16 st + 8 kb + i).
    u32x4 qop[G::DSTEPS];
    {
        const uint16_t* q = (const uint16_t*)a.q + ((int64_t)(valid ? r : 0) * H + h) * D;
#pragma unroll
        for (int st = 0; st < G::DSTEPS; ++st)
            qop[st] = valid ? *(const u32x4*)(q + 16 * st + 8 * kb) : u32x4{0u, 0u, 0u, 0u};
    }

    f32x16 O[G::DBLK];
#pragma unroll
    for (int db = 0; db < G::DBLK; ++db)
#pragma unroll
        for (int x = 0; x < 16; ++x)
            O[db][x] = 0.f;
    float m = neg_inf(), l = 0.f;
    const float sm_log2 = kLog2e / __builtin_sqrtf((float)D);

    if (tid == 0)
        s_bad = 0;
    int bad = 0;
    const uint8_t* kp = (const uint8_t*)a.k_pool;
    const uint8_t* vp = (const uint8_t*)a.v_pool;

    Stage<D, FP8> st;
    stage_load<D, FP8>(st, b, kp, vp, a.k_scale, a.v_scale, 0, tid, &bad);
    stage_store<D, FP8>(st, smem, tid);
    __syncthreads();

    for (int t = 0; t < nt; ++t) {
        const int tile0 = t * kKT;
        if (t + 1 < nt)
            stage_load<D, FP8>(st, b, kp, vp, a.k_scale, a.v_scale, tile0 + kKT, tid, &bad);
        const char* buf = smem + (t & 1) * G::BUF;
        const char* ks = buf;
        const char* vt = buf + G::KBYTES;
        const float* sc = (const float*)(buf + G::KBYTES + G::VBYTES);

        // S^T for the two 32-key blocks of the tile.
        f32x16 acc[2];
#pragma unroll
        for (int kblk = 0; kblk < 2; ++kblk) {
#pragma unroll
            for (int x = 0; x < 16; ++x)
                acc[kblk][x] = 0.f;
            const char* krow = ks + (32 * kblk + l32) * G::KS + 16 * kb;
#pragma unroll
            for (int s2 = 0; s2 < G::DSTEPS; ++s2) {
                const u32x4 kw = *(const u32x4*)(krow + 32 * s2);
                acc[kblk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, kw), __builtin_bit_cast(bf16x8, qop[s2]), acc[kblk],
                    0, 0, 0);
            }
        }

        // Scores, mask, online softmax (row = this lane's row).
        const bool diag = tile0 + kKT - 1 > minpos;
        float tmax = neg_inf();
#pragma unroll
        for (int kblk = 0; kblk < 2; ++kblk) {
            float s0 = sm_log2, s1 = sm_log2;
            if constexpr (FP8) {
                s0 = sc[2 * kblk] * sm_log2;
                s1 = sc[2 * kblk + 1] * sm_log2;
            }
#pragma unroll
            for (int x = 0; x < 16; ++x) {
                const int key = tile0 + 32 * kblk + 8 * (x >> 2) + 4 * kb + (x & 3);
                float v = acc[kblk][x] * ((x >> 3) ? s1 : s0);
                if (diag)
                    v = key <= pos ? v : neg_inf();
                acc[kblk][x] = v;
                tmax = fmaxf(tmax, v);
            }
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const float mnew = fmaxf(m, tmax);
        const float muse = mnew == neg_inf() ? 0.f : mnew;
        const float alpha = m == muse ? 1.f : __builtin_amdgcn_exp2f(m - muse);
        float psum = 0.f;
        u32x4 pb4[4];  // P^T operands of the 4 PV k-steps
#pragma unroll
        for (int kblk = 0; kblk < 2; ++kblk) {
            float vsc0 = 1.f, vsc1 = 1.f;
            if constexpr (FP8) {
                vsc0 = sc[4 + 2 * kblk];
                vsc1 = sc[4 + 2 * kblk + 1];
            }
            float pv[16];
#pragma unroll
            for (int x = 0; x < 16; ++x) {
                const float e = __builtin_amdgcn_exp2f(acc[kblk][x] - muse);
                psum = psum + e;
                pv[x] = FP8 ? e * ((x >> 3) ? vsc1 : vsc0) : e;
            }
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    pb4[2 * kblk + h2][w] = pack_bf16(pv[8 * h2 + 2 * w], pv[8 * h2 + 2 * w + 1]);
        }
        psum = psum + __shfl_xor(psum, 32, 64);
        l = l * alpha + psum;
        m = mnew;
        if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
            for (int db = 0; db < G::DBLK; ++db)
#pragma unroll
                for (int x = 0; x < 16; ++x)
                    O[db][x] = O[db][x] * alpha;
        }

        // O^T += V^T . P^T over the tile's 4 16-key steps.
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
#pragma unroll
            for (int db = 0; db < G::DBLK; ++db) {
                const char* vrow = vt + (32 * db + l32) * G::VS + (16 * s4 + 4 * kb) * 2;
                const u32x2 lo = *(const u32x2*)vrow;
                const u32x2 hi = *(const u32x2*)(vrow + 16);
                const u32x4 va = u32x4{lo[0], lo[1], hi[0], hi[1]};
                O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, va), __builtin_bit_cast(bf16x8, pb4[s4]), O[db], 0,
                    0, 0);
            }
        }

        if (t + 1 < nt)
            stage_store<D, FP8>(st, smem + ((t + 1) & 1) * G::BUF, tid);
        __syncthreads();
    }

    if (bad)
        s_bad = 1;
    __syncthreads();
    if (!valid)
        return;
    const bool nan = s_bad != 0;
    const float inv = 1.f / l;
    uint16_t* out = (uint16_t*)a.out + ((int64_t)r * H + h) * D;
#pragma unroll
    for (int db = 0; db < G::DBLK; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int d = 32 * db + 8 * q4 + 4 * kb;
            u32x2 o;
            o[0] = nan ? 0x7FC07FC0u : pack_bf16(O[db][4 * q4] * inv, O[db][4 * q4 + 1] * inv);
            o[1] = nan ? 0x7FC07FC0u : pack_bf16(O[db][4 * q4 + 2] * inv, O[db][4 * q4 + 3] * inv);
            *(u32x2*)(out + d) = o;
        }
}

template <int D, bool FP8>
hipError_t launch_t(const PrefillArgs& a, hipStream_t stream)
{
    const int g = a.n_head / a.n_head_kv;
    const int BP = 128 / g;
    const int npb = (a.n_rows + BP - 1) / BP;
    const int nblk = npb * a.n_head_kv;
    const int grid = ((nblk + 7) / 8) * 8;
    if (a.ev_start)
        (void)hipEventRecord(a.ev_start, stream);
    hipLaunchKernelGGL((prefill_kernel<D, FP8>), dim3(grid), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && a.ev_stop)
        (void)hipEventRecord(a.ev_stop, stream);
    return e;
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream)
{
    const int g = a.n_head / a.n_head_kv;
    if (g > 128 || 128 % g != 0)
        return hipErrorNotSupported;
    if (a.head_dim == 128)
        return a.fp8 ? launch_t<128, true>(a, stream) : launch_t<128, false>(a, stream);
    if (a.head_dim == 256)
        return a.fp8 ? launch_t<256, true>(a, stream) : launch_t<256, false>(a, stream);
    return hipErrorNotSupported;
}

}  // namespace pa
