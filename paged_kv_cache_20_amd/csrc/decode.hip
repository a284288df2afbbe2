// decode.hip -- split-K paged attention for the decode step (1 row per
// sequence) and the speculative verify round (8 rows per sequence), gfx950.
//
// Call shapes: "kern manifest v7" schema, $defs.Batch (rows 1 for a decode
// step, exactly 8 for a speculative round); row r of a call with R rows sits
// at position ctx_len - R + r ($defs.Fill "seq_len" counts the call's rows).
//
// Work decomposition
//   A work item is (sequence s, split j, kv head kh): keys [512 j, 512 j + 512)
//   of s, clipped to ctx_len.  Split boundaries are absolute multiples of 512,
//   so the items a row takes part in, and everything computed inside them,
//   depend on the row's position and its sequence's own data only.  Each wave
//   of a persistent grid walks items (wave, wave + total waves, ...); which
//   wave takes an item changes nothing in its arithmetic.
//
// Inside an item (one 64-lane wave)
//   Query rows are packed into 16-slot MFMA tiles.  A tile holds floor(16/g)
//   positions x g heads of the kv group (g = n_head / n_head_kv); position p
//   and head-in-group c sit in slot g * (p mod floor(16/g)) + c, so a
//   position occupies the same MFMA column in a decode call and in a verify
//   call.  Keys stream in tiles of 32 (two 16-token pages):
//     S^T[key][slot] = K . Q^T     v_mfma_f32_16x16x32_bf16, keys as rows
//     online softmax per slot      exp2, max/sum across the wave's 4 k-groups
//     O[slot][d]    += P . V       v_mfma_f32_16x16x32_bf16
//   The S^T accumulator layout (lane = slot + 16 * key group) is exactly the
//   A-operand layout P needs, so P never moves between lanes.  K is read in
//   A-operand order (16-byte pieces, one key row per lane); V is read
//   row-contiguous (each 16 lanes cover whole token rows) and transposed in
//   registers with byte permutes.  fp8 codes become bf16 exactly in
//   registers; the K scale multiplies the scores, the V scale is folded into
//   P, both per page.
//   Keys at or beyond ctx_len are never loaded (zeros take their place) and
//   are masked; a fully masked tile leaves m, l and O bit-identical.
//
// Combine: per (sequence, row, head), splits 0 .. floor(pos / 512) are merged
// in increasing order: M = max m_j, w_j = exp2(m_j - M),
// out = sum w_j o_j / sum w_j l_j, rounded to bf16.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;  // waves per block
constexpr int kKT = 32;    // keys per inner tile
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }

__device__ __forceinline__ uint32_t bf16_bits(float x)
{
    __bf16 b = (__bf16)x;  // round to nearest even
    return (uint32_t)__builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    return bf16_bits(lo) | (bf16_bits(hi) << 16);
}

// Two e4m3 codes (bytes 2*hi, 2*hi+1 of w) -> two bf16, exact.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w)
{
    bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HI);
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ int shfl_xor_i(int v, int m) { return __shfl_xor(v, m, 64); }
__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

template <int D, bool FP8>
struct Geo {
    static constexpr int EB = FP8 ? 1 : 2;      // bytes per stored element
    static constexpr int ROWB = D * EB;         // bytes per token row of one kv head
    static constexpr int STEPS = D / 32;        // k-steps of the QK^T contraction
    static constexpr int KLD = ROWB / 64;       // 16-byte K loads per lane per key block
    static constexpr int VPB = ROWB / 16;       // V bytes per lane per token
    static constexpr int VDW = VPB / 4;         // ... in dwords
    static constexpr int DB = D / 16;           // output columns per lane (d blocks)
    static constexpr int RAW = 2 * KLD * 4 + 8 * VDW;  // raw tile dwords per lane
};

template <int D, bool FP8>
struct Raw {
    u32x4 k[2][Geo<D, FP8>::KLD];
    uint32_t v[8][Geo<D, FP8>::VDW];
};

// Element offset (in the query row) of the first of the 8 d-values that
// lane group kb feeds into k-step st.  Matches the K read order below.
template <int D, bool FP8>
__device__ __forceinline__ int qk_dmap(int st, int kb)
{
    if (FP8)
        return 64 * (st >> 1) + 16 * kb + 8 * (st & 1);
    return 32 * st + 8 * kb;
}

// K A-operand of k-step st from a lane's raw K pieces (8 bf16).
template <int D, bool FP8>
__device__ __forceinline__ bf16x8 k_operand(const u32x4* kr, int st)
{
    if constexpr (FP8) {
        const u32x4 w = kr[st >> 1];
        const uint32_t lo = (st & 1) ? w[2] : w[0];
        const uint32_t hi = (st & 1) ? w[3] : w[1];
        u32x4 o;
        o[0] = fp8x2_to_bf16x2<false>(lo);
        o[1] = fp8x2_to_bf16x2<true>(lo);
        o[2] = fp8x2_to_bf16x2<false>(hi);
        o[3] = fp8x2_to_bf16x2<true>(hi);
        return __builtin_bit_cast(bf16x8, o);
    } else {
        return __builtin_bit_cast(bf16x8, kr[st]);
    }
}

// Key (within the 32-key tile) that lane group kb feeds at k-slot i of the
// PV product; the same keys the lane holds in its S^T accumulators.
__device__ __forceinline__ int pv_key(int kb, int i) { return i < 4 ? 4 * kb + i : 12 + 4 * kb + i; }

template <int D, bool FP8>
__device__ __forceinline__ void load_tile(Raw<D, FP8>& t, const uint8_t* __restrict__ kp,
                                          const uint8_t* __restrict__ vp, int pg0, int pg1,
                                          int kt, int C, int Hk, int kh, int n, int kb)
{
    using G = Geo<D, FP8>;
#pragma unroll
    for (int kblk = 0; kblk < 2; ++kblk) {
        const int key = kt + 16 * kblk + n;
        const int pg = kblk ? pg1 : pg0;
        if (key < C) {
            const uint8_t* row = kp + (((int64_t)pg * Hk + kh) * 16 + n) * G::ROWB + 16 * kb;
#pragma unroll
            for (int c = 0; c < G::KLD; ++c)
                t.k[kblk][c] = *(const u32x4*)(row + 64 * c);
        } else {
#pragma unroll
            for (int c = 0; c < G::KLD; ++c)
                t.k[kblk][c] = u32x4{0u, 0u, 0u, 0u};
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int kk = pv_key(kb, i);
        const int key = kt + kk;
        const int pg = (kk >> 4) ? pg1 : pg0;
        if (key < C) {
            const uint8_t* row =
                vp + (((int64_t)pg * Hk + kh) * 16 + (kk & 15)) * G::ROWB + n * G::VPB;
            if constexpr (G::VDW == 2) {
                const u32x2 w = *(const u32x2*)row;
                t.v[i][0] = w[0];
                t.v[i][1] = w[1];
            } else {
#pragma unroll
                for (int c = 0; c < G::VDW / 4; ++c) {
                    const u32x4 w = *(const u32x4*)(row + 16 * c);
                    t.v[i][4 * c + 0] = w[0];
                    t.v[i][4 * c + 1] = w[1];
                    t.v[i][4 * c + 2] = w[2];
                    t.v[i][4 * c + 3] = w[3];
                }
            }
        } else {
#pragma unroll
            for (int c = 0; c < G::VDW; ++c)
                t.v[i][c] = 0u;
        }
    }
}

// Row held by slot `slot` of tile `tau` (-1 if the slot is empty).
__device__ __forceinline__ int slot_row(int slot, int tau, int g, int ppt, int R, int cmr_mod)
{
    const int pp = slot / g;
    if (pp >= ppt)
        return -1;
    const int u = (pp - cmr_mod + ppt) % ppt;
    const int r = tau * ppt + u;
    return r < R ? r : -1;
}

template <int D, bool FP8, int NT>
__device__ __forceinline__ void compute_tile(const Raw<D, FP8>& t, const u32x4 (&qop)[NT][D / 32],
                                             const int (&last)[NT], float (&m)[NT], float (&l)[NT],
                                             f32x4 (&O)[NT][D / 16], int kt, float sc0, float sc1,
                                             float vs0, float vs1, int lane, int kb)
{
    using G = Geo<D, FP8>;
    f32x4 acc[2][NT];
#pragma unroll
    for (int kblk = 0; kblk < 2; ++kblk)
#pragma unroll
        for (int tau = 0; tau < NT; ++tau)
            acc[kblk][tau] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < G::STEPS; ++st) {
#pragma unroll
        for (int kblk = 0; kblk < 2; ++kblk) {
            const bf16x8 ka = k_operand<D, FP8>(t.k[kblk], st);
#pragma unroll
            for (int tau = 0; tau < NT; ++tau)
                acc[kblk][tau] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    ka, __builtin_bit_cast(bf16x8, qop[tau][st]), acc[kblk][tau], 0, 0, 0);
        }
    }

    u32x4 pa[NT];
    float alpha[NT];
#pragma unroll
    for (int tau = 0; tau < NT; ++tau) {
        float sv[2][4];
        float tmax = neg_inf();
#pragma unroll
        for (int kblk = 0; kblk < 2; ++kblk)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = kt + 16 * kblk + 4 * kb + r;
                const float x = acc[kblk][tau][r] * (kblk ? sc1 : sc0);
                sv[kblk][r] = key <= last[tau] ? x : neg_inf();
                tmax = fmaxf(tmax, sv[kblk][r]);
            }
        tmax = fmaxf(tmax, shfl_xor_f(tmax, 16));
        tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
        const float mnew = fmaxf(m[tau], tmax);
        const float muse = mnew == neg_inf() ? 0.f : mnew;
        const float al = m[tau] == muse ? 1.f : __builtin_amdgcn_exp2f(m[tau] - muse);
        float p[2][4];
#pragma unroll
        for (int kblk = 0; kblk < 2; ++kblk)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                p[kblk][r] = __builtin_amdgcn_exp2f(sv[kblk][r] - muse);
        float psum = ((p[0][0] + p[0][1]) + (p[0][2] + p[0][3])) +
                     ((p[1][0] + p[1][1]) + (p[1][2] + p[1][3]));
        psum = psum + shfl_xor_f(psum, 16);
        psum = psum + shfl_xor_f(psum, 32);
        l[tau] = l[tau] * al + psum;
        m[tau] = mnew;
        alpha[tau] = al;
        if constexpr (FP8) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                p[0][r] = p[0][r] * vs0;
                p[1][r] = p[1][r] * vs1;
            }
        }
        pa[tau][0] = pack_bf16(p[0][0], p[0][1]);
        pa[tau][1] = pack_bf16(p[0][2], p[0][3]);
        pa[tau][2] = pack_bf16(p[1][0], p[1][1]);
        pa[tau][3] = pack_bf16(p[1][2], p[1][3]);
    }

    // Rescale O rows (slot 4*kb + r) by their slot's alpha; skipping a
    // multiply by exactly 1 changes nothing.
#pragma unroll
    for (int tau = 0; tau < NT; ++tau) {
        if (__builtin_amdgcn_ballot_w64(alpha[tau] != 1.f)) {
            float ar[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                ar[r] = __shfl(alpha[tau], 4 * kb + r, 64);
#pragma unroll
            for (int jb = 0; jb < G::DB; ++jb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    O[tau][jb][r] = O[tau][jb][r] * ar[r];
        }
    }

    // V B-operands: column n of d-block jb is d = n * DB + jb; k-slot i is
    // token pv_key(kb, i).
    uint32_t vb[8][G::DB / 2];  // bf16 pieces: token i, dword w = elements 2w, 2w+1
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if constexpr (FP8) {
#pragma unroll
            for (int w = 0; w < G::VDW; ++w) {
                vb[i][2 * w] = fp8x2_to_bf16x2<false>(t.v[i][w]);
                vb[i][2 * w + 1] = fp8x2_to_bf16x2<true>(t.v[i][w]);
            }
        } else {
#pragma unroll
            for (int w = 0; w < G::VDW; ++w)
                vb[i][w] = t.v[i][w];
        }
    }
#pragma unroll
    for (int jb = 0; jb < G::DB; ++jb) {
        const uint32_t sel = (jb & 1) ? 0x07060302u : 0x05040100u;
        u32x4 b;
#pragma unroll
        for (int u = 0; u < 4; ++u)
            b[u] = __builtin_amdgcn_perm(vb[2 * u + 1][jb >> 1], vb[2 * u][jb >> 1], sel);
#pragma unroll
        for (int tau = 0; tau < NT; ++tau)
            O[tau][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, pa[tau]), __builtin_bit_cast(bf16x8, b), O[tau][jb], 0,
                0, 0);
    }
    (void)lane;
}

__device__ __forceinline__ bool ctx_ok(int C, int R, int64_t cap) { return C >= R && (int64_t)C <= cap; }

template <int D, bool FP8, int NT>
__global__ __launch_bounds__(256) void split_kernel(SplitArgs a)
{
    using G = Geo<D, FP8>;
    constexpr bool DBUF = 2 * G::RAW + NT * (G::STEPS + G::DB) * 4 <= 256;
    __shared__ int s_pre[kMaxSeq + 1];
    __shared__ int s_tmp[256];

    const int S = a.n_seq, R = a.rows, Hk = a.n_head_kv, H = a.n_head;
    const int g = H / Hk, ppt = 16 / g;
    const int64_t cap = (int64_t)a.max_pages * 16;
    const int tid = threadIdx.x;

    // Exclusive prefix over sequences of their work items.
    {
        const int per = (S + 255) / 256;
        const int b0 = tid * per;
        int loc = 0;
        for (int i = 0; i < per; ++i) {
            const int s = b0 + i;
            if (s < S) {
                const int C = a.ctx_lens[s];
                loc += ctx_ok(C, R, cap) ? ((C + kChunk - 1) / kChunk) * Hk : 0;
            }
        }
        s_tmp[tid] = loc;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const int v = tid >= off ? s_tmp[tid - off] : 0;
            __syncthreads();
            s_tmp[tid] += v;
            __syncthreads();
        }
        int run = tid ? s_tmp[tid - 1] : 0;
        for (int i = 0; i < per; ++i) {
            const int s = b0 + i;
            if (s < S) {
                s_pre[s] = run;
                const int C = a.ctx_lens[s];
                run += ctx_ok(C, R, cap) ? ((C + kChunk - 1) / kChunk) * Hk : 0;
            }
        }
        if (tid == 255)
            s_pre[S] = s_tmp[255];
        __syncthreads();
    }

    const int lane = tid & 63, n = lane & 15, kb = lane >> 4;
    const int total = s_pre[S];
    const int nwaves = gridDim.x * kWaves;
    const float sm_log2 = kLog2e / __builtin_sqrtf((float)D);
    const uint8_t* __restrict__ kp = (const uint8_t*)a.k_pool;
    const uint8_t* __restrict__ vp = (const uint8_t*)a.v_pool;

    for (int item = blockIdx.x * kWaves + (tid >> 6); item < total; item += nwaves) {
        int lo = 0, hi = S - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_pre[mid] <= item)
                lo = mid;
            else
                hi = mid - 1;
        }
        const int s = __builtin_amdgcn_readfirstlane(lo);
        const int local = item - s_pre[s];
        const int j = local / Hk, kh = local - j * Hk;
        const int C = a.ctx_lens[s];
        const int t0 = j * kChunk;
        const int t1 = min(t0 + kChunk, C);
        const int cmr_mod = (C - R) % ppt;

        // Pages of this item: lane i holds entry i (and its scales).
        const int npg = (t1 - t0 + 15) >> 4;
        int pid = -1;
        float ksc = 0.f, vsc = 0.f;
        if (lane < npg)
            pid = a.block_table[(int64_t)s * a.max_pages + (t0 >> 4) + lane];
        const bool badp = lane < npg && (pid < 0 || (int64_t)pid >= a.n_pages);
        const bool bad = __builtin_amdgcn_ballot_w64(badp) != 0;
        if (!bad && FP8 && lane < npg) {
            ksc = a.k_scale[(int64_t)pid * Hk + kh];
            vsc = a.v_scale[(int64_t)pid * Hk + kh];
        }

        u32x4 qop[NT][G::STEPS];
        int last[NT];
        float m[NT], l[NT];
        f32x4 O[NT][G::DB];
#pragma unroll
        for (int tau = 0; tau < NT; ++tau) {
            const int r = slot_row(n, tau, g, ppt, R, cmr_mod);
            last[tau] = r >= 0 ? C - R + r : -1;
            const int h = kh * g + (n % g);
            const uint16_t* qrow =
                (const uint16_t*)a.q + (((int64_t)s * R + (r >= 0 ? r : 0)) * H + h) * D;
#pragma unroll
            for (int st = 0; st < G::STEPS; ++st)
                qop[tau][st] = r >= 0 ? *(const u32x4*)(qrow + qk_dmap<D, FP8>(st, kb))
                                      : u32x4{0u, 0u, 0u, 0u};
            m[tau] = neg_inf();
            l[tau] = 0.f;
#pragma unroll
            for (int jb = 0; jb < G::DB; ++jb)
                O[tau][jb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

        if (!bad) {
            const int nt = (t1 - t0 + kKT - 1) / kKT;
            auto page = [&](int e) { return e < npg ? __shfl(pid, e, 64) : 0; };
            auto kscale = [&](int e) { return FP8 ? __shfl(ksc, e, 64) * sm_log2 : sm_log2; };
            auto vscale = [&](int e) { return FP8 ? __shfl(vsc, e, 64) : 1.f; };
            if constexpr (DBUF) {
                Raw<D, FP8> A, B;
                load_tile<D, FP8>(A, kp, vp, page(0), page(1), t0, C, Hk, kh, n, kb);
                for (int it = 0; it < nt; it += 2) {
                    if (it + 1 < nt)
                        load_tile<D, FP8>(B, kp, vp, page(2 * it + 2), page(2 * it + 3),
                                          t0 + kKT * (it + 1), C, Hk, kh, n, kb);
                    compute_tile<D, FP8, NT>(A, qop, last, m, l, O, t0 + kKT * it,
                                             kscale(2 * it), kscale(2 * it + 1), vscale(2 * it),
                                             vscale(2 * it + 1), lane, kb);
                    if (it + 1 < nt) {
                        if (it + 2 < nt)
                            load_tile<D, FP8>(A, kp, vp, page(2 * it + 4), page(2 * it + 5),
                                              t0 + kKT * (it + 2), C, Hk, kh, n, kb);
                        compute_tile<D, FP8, NT>(B, qop, last, m, l, O, t0 + kKT * (it + 1),
                                                 kscale(2 * it + 2), kscale(2 * it + 3),
                                                 vscale(2 * it + 2), vscale(2 * it + 3), lane, kb);
                    }
                }
            } else {
                Raw<D, FP8> A;
                for (int it = 0; it < nt; ++it) {
                    load_tile<D, FP8>(A, kp, vp, page(2 * it), page(2 * it + 1), t0 + kKT * it, C,
                                      Hk, kh, n, kb);
                    compute_tile<D, FP8, NT>(A, qop, last, m, l, O, t0 + kKT * it,
                                             kscale(2 * it), kscale(2 * it + 1), vscale(2 * it),
                                             vscale(2 * it + 1), lane, kb);
                }
            }
        }

        // Partials: O rows are slots 4*kb + r; m, l of slot n.
        const float qnan = __builtin_nanf("");
#pragma unroll
        for (int tau = 0; tau < NT; ++tau) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int slot = 4 * kb + r;
                const int row = slot_row(slot, tau, g, ppt, R, cmr_mod);
                if (row >= 0) {
                    const int h = kh * g + (slot % g);
                    float* dst = a.o_part +
                                 ((((int64_t)s * a.max_split + j) * R + row) * H + h) * D + n * G::DB;
#pragma unroll
                    for (int jb = 0; jb < G::DB; jb += 4)
                        *(f32x4*)(dst + jb) =
                            bad ? f32x4{qnan, qnan, qnan, qnan}
                                : f32x4{O[tau][jb][r], O[tau][jb + 1][r], O[tau][jb + 2][r],
                                        O[tau][jb + 3][r]};
                }
            }
            const int row = slot_row(n, tau, g, ppt, R, cmr_mod);
            if (kb == 0 && row >= 0) {
                const int h = kh * g + (n % g);
                float* dst = a.ml_part + ((((int64_t)s * a.max_split + j) * R + row) * H + h) * 2;
                dst[0] = bad ? qnan : m[tau];
                dst[1] = bad ? qnan : l[tau];
            }
        }
    }
}

// One wave per (sequence, row, head); lanes own D/64 consecutive d-values.
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(SplitArgs a)
{
    constexpr int E = D / 64;
    const int lane = threadIdx.x & 63;
    const int64_t w = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    const int R = a.rows, H = a.n_head;
    if (w >= (int64_t)a.n_seq * R * H)
        return;
    const int h = (int)(w % H);
    const int64_t sr = w / H;
    const int r = (int)(sr % R), s = (int)(sr / R);
    const int C = a.ctx_lens[s];
    uint16_t* out = (uint16_t*)a.out + w * D + lane * E;
    const int64_t cap = (int64_t)a.max_pages * 16;
    if (!ctx_ok(C, R, cap)) {
#pragma unroll
        for (int e = 0; e < E; ++e)
            out[e] = 0x7FC0;  // NaN
        return;
    }
    const int pos = C - R + r;
    const int ns = pos / kChunk + 1;
    const float* ml = a.ml_part + (((int64_t)s * a.max_split * R + r) * H + h) * 2;
    const float* op = a.o_part + (((int64_t)s * a.max_split * R + r) * H + h) * D + lane * E;
    const int64_t mls = (int64_t)R * H * 2, ops = (int64_t)R * H * D;  // per-split strides

    float M = neg_inf();
    bool nan = false;
    for (int j = 0; j < ns; ++j) {
        const float mj = ml[j * mls];
        nan |= mj != mj;
        M = fmaxf(M, mj);
    }
    float num[E], den = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e)
        num[e] = 0.f;
    for (int j = 0; j < ns; ++j) {
        const float mj = ml[j * mls], lj = ml[j * mls + 1];
        const float wj = mj == M ? 1.f : __builtin_amdgcn_exp2f(mj - M);
        den = den + wj * lj;
        const float* oj = op + j * ops;
#pragma unroll
        for (int e = 0; e < E; ++e)
            num[e] = num[e] + wj * oj[e];
    }
#pragma unroll
    for (int e = 0; e < E; ++e)
        out[e] = nan ? (uint16_t)0x7FC0 : (uint16_t)bf16_bits(num[e] / den);
}

template <int D, bool FP8, int NT>
hipError_t launch_split_t(const SplitArgs& a, hipStream_t stream)
{
    static int s_grid[64] = {0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    int& grid_cap = s_grid[dev & 63];
    if (grid_cap == 0) {
        int cus = 0, per = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess)
            return e;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, split_kernel<D, FP8, NT>, 256, 0);
        if (e != hipSuccess)
            return e;
        grid_cap = cus * (per > 0 ? per : 1);
    }
    const int Hk = a.n_head_kv;
    const int64_t upper = (int64_t)a.n_seq * a.max_split * Hk;  // items, at most
    int64_t blocks = (upper + kWaves - 1) / kWaves;
    if (blocks > grid_cap)
        blocks = grid_cap;
    if (blocks < 1)
        blocks = 1;
    if (a.ev_start)
        (void)hipEventRecord(a.ev_start, stream);
    hipLaunchKernelGGL((split_kernel<D, FP8, NT>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    if (a.ev_stop)
        (void)hipEventRecord(a.ev_stop, stream);
    const int64_t waves = (int64_t)a.n_seq * a.rows * a.n_head;
    hipLaunchKernelGGL((combine_kernel<D>), dim3((unsigned)((waves + kWaves - 1) / kWaves)),
                       dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <int D, bool FP8>
hipError_t launch_nt(const SplitArgs& a, int nt, hipStream_t stream)
{
    switch (nt) {
    case 1: return launch_split_t<D, FP8, 1>(a, stream);
    case 2: return launch_split_t<D, FP8, 2>(a, stream);
    case 4:
        if constexpr (D <= 128)
            return launch_split_t<D, FP8, 4>(a, stream);
        return hipErrorNotSupported;
    default: return hipErrorNotSupported;
    }
}

}  // namespace

// Tiles of 16 slots a call needs: ceil(rows / floor(16 / g)), rounded up to
// an instantiated count.
int split_tiles(int rows, int g)
{
    const int ppt = 16 / g;
    const int t = (rows + ppt - 1) / ppt;
    return t <= 1 ? 1 : t <= 2 ? 2 : t <= 4 ? 4 : 8;
}

hipError_t launch_split_decode(const SplitArgs& a, hipStream_t stream)
{
    const int g = a.n_head / a.n_head_kv;
    const int nt = split_tiles(a.rows, g);
    if (a.head_dim == 128)
        return a.fp8 ? launch_nt<128, true>(a, nt, stream) : launch_nt<128, false>(a, nt, stream);
    if (a.head_dim == 256)
        return a.fp8 ? launch_nt<256, true>(a, nt, stream) : launch_nt<256, false>(a, nt, stream);
    return hipErrorNotSupported;
}

}  // namespace pa
