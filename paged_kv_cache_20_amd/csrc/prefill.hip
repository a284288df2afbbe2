// prefill.hip -- a chunk of new rows of ONE sequence over its paged cache
// ("kern manifest v7" schema, $defs.Batch: one sequence, as many rows as the
// chunk; `context` is the cached rows the call expands over).  Row r of an
// n_rows chunk sits at position ctx_len - n_rows + r and attends to keys
// 0 .. that position.
//
// Work decomposition (gfx950)
//   A workgroup of 8 waves owns one kv head and 128 query rows: 128/g
//   consecutive positions x the g query heads that share the kv head, so
//   every K/V tile it stages serves g heads.  Wave w owns rows 16w..16w+15,
//   which keeps a wave's Q (32 VGPRs) and O (64 accumulators) small enough
//   for two waves per SIMD: one wave's matrix work overlaps the other's
//   softmax.
//   Keys stream in 64-key tiles (four 16-token pages) through two LDS
//   buffers, K and V both row-major as bf16 with each row's 16-byte chunks
//   XOR-swizzled by the row index (conflict-free reads of a column of rows).
//   bf16 pages are copied global -> LDS by buffer loads that write LDS
//   directly (no registers in flight); the buffer descriptor of each page
//   covers only the rows below ctx_len, so rows past the context arrive as
//   zeros.  fp8 pages are loaded into registers, converted to bf16 exactly
//   and written to the same layout.
//   Per wave and tile, on v_mfma_f32_16x16x32_bf16:
//     S^T[key][row] = K . Q^T      K rows by ds_read_b128, Q^T in registers
//     online softmax               a row's 16 scores of the tile sit in the 4
//                                  lanes row + 16 j, so max and sum take two
//                                  cross-lane swaps
//     O^T[d][row]  += V^T . P^T    V^T by ds_read_b64_tr_b16 (a 4-key x
//                                  16-column block per 16 lanes, transposed
//                                  in the read); P^T is the S^T accumulator
//                                  re-packed in place; O^T's row is again
//                                  the lane's row, so rescaling and 1/l are
//                                  lane-local
//   The row max only moves when a score of the tile exceeds it by more than
//   2^8 (checked once per tile, before any of its scores becomes a
//   probability), so O is rarely rescaled (P stays <= 2^8).
//   Workgroups of one kv head are placed on the same XCDs (blockIdx mod 8
//   picks the XCD) so the K/V tiles they stream share that XCD's L2.
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
typedef short s16x4 __attribute__((ext_vector_type(4)));

#define LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kKT = 64;       // keys per tile
constexpr int kWaves = 8;     // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr float kTau = 8.f;   // lazy-rescale threshold (log2 units)
constexpr int kRsrcFlags = 0x00020000;

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

// Physical 16-byte chunk of logical chunk c in LDS row r is c ^ swz(r).
// swz is one-to-one on r's low four bits, one-to-one modulo 8 on any 8
// aligned rows, and spreads {c, c+1} (c even) of any 4 (8) aligned rows over
// 8 (16) different chunks: the K reads (16 rows, one chunk) and the V reads
// (4 rows per 16 lanes, two chunks) are conflict-free whether the LDS serves
// 128 or 256 bytes per clock.
__device__ __forceinline__ int swz(int r)
{
    return ((r >> 2) & 1) | ((r & 1) << 1) | (((r >> 1) & 1) << 2) |
           ((((r >> 2) ^ (r >> 3)) & 1) << 3);
}

template <int D, bool FP8>
struct PGeo {
    static constexpr int EB = FP8 ? 1 : 2;
    static constexpr int ROWB = D * EB;          // bytes of one token row in the pool
    static constexpr int ROWL = D * 2;           // bytes of one row in LDS (bf16)
    static constexpr int CPRL = ROWL / 16;       // 16-byte chunks per LDS row
    static constexpr int TILEB = kKT * ROWL;     // one K (or V) tile in LDS
    static constexpr int BUF = 2 * TILEB + 64;   // K, V, per-page scales
    static constexpr int KSTEPS = D / 32;        // k-steps of QK^T
    static constexpr int DBLK = D / 16;          // 16-wide d blocks of O^T
    // direct (bf16) loads: 1 KiB LDS blocks
    static constexpr int RPB = 1024 / ROWL;            // rows per block
    static constexpr int NBW = (kKT / RPB) / kWaves;   // blocks per wave per tensor
    // staged (fp8) loads: 16-byte pool chunks per thread per tensor
    static constexpr int CPR = ROWB / 16;
    static constexpr int SCH = kKT * CPR / kThreads;
};

struct Blk {
    int C, kh, Hk;
    int64_t n_pages;
    const int32_t* bt;
};

// Block-table entries of the tile at tile0 (raw, not yet checked); -1 past
// the context.  Issued a tile ahead so their latency hides behind compute.
__device__ __forceinline__ void fetch_pages(const Blk& b, int tile0, int (&raw)[4])
{
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int key0 = tile0 + 16 * q;
        raw[q] = key0 < b.C ? b.bt[key0 >> 4] : -1;
    }
}

// Page of the q-th 16-key group of the tile at tile0 and the number of its
// rows below the context; page -1 (and 0 rows) past the context or for an
// entry outside the pool (which also raises *bad).
__device__ __forceinline__ void resolve_pages(const Blk& b, int tile0, const int (&raw)[4],
                                              int (&pg)[4], int (&rows)[4], int* bad)
{
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int key0 = tile0 + 16 * q;
        const int p = __builtin_amdgcn_readfirstlane(raw[q]);
        pg[q] = -1;
        rows[q] = 0;
        if (key0 < b.C) {
            if (p < 0 || (int64_t)p >= b.n_pages) {
                *bad = 1;
            } else {
                pg[q] = p;
                rows[q] = min(16, b.C - key0);
            }
        }
    }
}

// bf16: every wave issues its share of the tile's 1 KiB blocks as buffer
// loads that write LDS directly.
template <int D>
__device__ __forceinline__ void issue_direct(char* kbuf, char* vbuf, const Blk& b,
                                             const uint8_t* kp, const uint8_t* vp, int tile0,
                                             int wave, const int (&loff)[PGeo<D, false>::NBW],
                                             const int (&raw)[4], int* bad)
{
    using G = PGeo<D, false>;
    int pg[4], rows[4];
    resolve_pages(b, tile0, raw, pg, rows, bad);
#pragma unroll
    for (int i = 0; i < G::NBW; ++i) {
        const int blk = wave * G::NBW + i;
        const int q = (blk * G::RPB) >> 4;
        const int64_t base = ((int64_t)(pg[q] < 0 ? 0 : pg[q]) * b.Hk + b.kh) * 16 * G::ROWB;
        const int nrec = rows[q] * G::ROWB;
        __amdgpu_buffer_rsrc_t rk =
            __builtin_amdgcn_make_buffer_rsrc((void*)(kp + base), (short)0, nrec, kRsrcFlags);
        __amdgpu_buffer_rsrc_t rv =
            __builtin_amdgcn_make_buffer_rsrc((void*)(vp + base), (short)0, nrec, kRsrcFlags);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (LDS void*)(kbuf + blk * 1024), 16, loff[i],
                                                 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (LDS void*)(vbuf + blk * 1024), 16, loff[i],
                                                 0, 0, 0);
    }
}

// fp8: a thread's share of the tile in registers between load and store.
template <int D>
struct Staged {
    u32x4 k[PGeo<D, true>::SCH];
    u32x4 v[PGeo<D, true>::SCH];
    float ks, vs;
};

template <int D>
__device__ __forceinline__ void stage_load(Staged<D>& st, const Blk& b, const uint8_t* kp,
                                           const uint8_t* vp, const float* ksc, const float* vsc,
                                           int tile0, int tid, int* bad)
{
    using G = PGeo<D, true>;
    int pg[4], rows[4], raw[4];
    fetch_pages(b, tile0, raw);
    resolve_pages(b, tile0, raw, pg, rows, bad);
#pragma unroll
    for (int i = 0; i < G::SCH; ++i) {
        const int c = i * kThreads + tid;
        const int key = c / G::CPR, piece = c % G::CPR;
        const int q = key >> 4;
        if ((key & 15) < rows[q]) {
            const int64_t off =
                (((int64_t)pg[q] * b.Hk + b.kh) * 16 + (key & 15)) * G::ROWB + piece * 16;
            st.k[i] = *(const u32x4*)(kp + off);
            st.v[i] = *(const u32x4*)(vp + off);
        } else {
            st.k[i] = u32x4{0u, 0u, 0u, 0u};
            st.v[i] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    if (tid < 4) {  // pages past the context: scale 1 (their keys are masked)
        st.ks = pg[tid] >= 0 ? ksc[(int64_t)pg[tid] * b.Hk + b.kh] : 1.f;
        st.vs = pg[tid] >= 0 ? vsc[(int64_t)pg[tid] * b.Hk + b.kh] : 1.f;
    }
}

template <int D>
__device__ __forceinline__ void stage_store(const Staged<D>& st, char* kbuf, char* vbuf,
                                            float* sc, int tid)
{
    using G = PGeo<D, true>;
#pragma unroll
    for (int i = 0; i < G::SCH; ++i) {
        const int c = i * kThreads + tid;
        const int key = c / G::CPR, piece = c % G::CPR;
#pragma unroll
        for (int kv = 0; kv < 2; ++kv) {
            const u32x4 w = kv ? st.v[i] : st.k[i];
            char* row = (kv ? vbuf : kbuf) + key * G::ROWL;
            u32x4 lo, hi;
            lo[0] = fp8x2_to_bf16x2<false>(w[0]);
            lo[1] = fp8x2_to_bf16x2<true>(w[0]);
            lo[2] = fp8x2_to_bf16x2<false>(w[1]);
            lo[3] = fp8x2_to_bf16x2<true>(w[1]);
            hi[0] = fp8x2_to_bf16x2<false>(w[2]);
            hi[1] = fp8x2_to_bf16x2<true>(w[2]);
            hi[2] = fp8x2_to_bf16x2<false>(w[3]);
            hi[3] = fp8x2_to_bf16x2<true>(w[3]);
            *(u32x4*)(row + ((2 * piece) ^ swz(key)) * 16) = lo;
            *(u32x4*)(row + ((2 * piece + 1) ^ swz(key)) * 16) = hi;
        }
    }
    if (tid < 4) {
        sc[tid] = st.ks;
        sc[4 + tid] = st.vs;
    }
}

template <int D, bool FP8>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillArgs a)
{
    using G = PGeo<D, FP8>;
    __shared__ __attribute__((aligned(1024))) char smem0[G::BUF];
    __shared__ __attribute__((aligned(1024))) char smem1[G::BUF];
    __shared__ int s_bad;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
    const int n = lane & 15, kb = lane >> 4;
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
    b.kh = kh;
    b.Hk = Hk;
    b.n_pages = a.n_pages;
    b.bt = a.block_table;
    const int base_pos = a.ctx_len - a.n_rows;

    // This lane's query row (row n of the wave's 16).
    const int wrow = 16 * wave + n;            // 0..127 in the workgroup
    const int hg = wrow / BP, p = wrow - hg * BP;
    const int r = pb * BP + p;                 // row of the call
    const bool valid = r < a.n_rows;
    const int h = kh * g + hg;
    const int pos = valid ? base_pos + r : -1;
    const int rlast = min(a.n_rows, (pb + 1) * BP) - 1;
    const int maxpos = base_pos + rlast;       // last key any row here needs
    const int minpos = base_pos + pb * BP;
    const int nt = (maxpos + kKT) / kKT;

    // Q^T operand: 8 bf16 of the lane's row per k-step (d = 32 st + 8 kb + i).
    u32x4 qop[G::KSTEPS];
    {
        const uint16_t* q = (const uint16_t*)a.q + ((int64_t)(valid ? r : 0) * H + h) * D;
#pragma unroll
        for (int st = 0; st < G::KSTEPS; ++st)
            qop[st] = valid ? *(const u32x4*)(q + 32 * st + 8 * kb) : u32x4{0u, 0u, 0u, 0u};
    }

    f32x4 O[G::DBLK];
#pragma unroll
    for (int jb = 0; jb < G::DBLK; ++jb)
        O[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = neg_inf(), l = 0.f;
    const float sm_log2 = kLog2e / __builtin_sqrtf((float)D);

    if (tid == 0)
        s_bad = 0;
    int bad = 0;
    const uint8_t* kp = (const uint8_t*)a.k_pool;
    const uint8_t* vp = (const uint8_t*)a.v_pool;

    // Per-lane byte offsets, fixed for the whole call.
    // Direct loads: instruction i of this wave fills LDS block wave*NBW + i;
    // this lane writes row rr, physical chunk pc of it and so fetches
    // logical chunk pc ^ swz(row) of that row.
    int loff[G::NBW];
    if constexpr (!FP8) {
        const int rr = lane / G::CPRL, pc = lane % G::CPRL;
#pragma unroll
        for (int i = 0; i < G::NBW; ++i) {
            const int row = (wave * G::NBW + i) * G::RPB + rr;
            loff[i] = (row & 15) * G::ROWB + ((pc ^ swz(row)) * 16);
        }
    }
    // K reads: key row 16 kq + n (kq = 16-key block), logical chunk 4 st + kb.
    // swz(16 kq + n) = swz(n), and it touches the low 4 chunk bits, so a read
    // = base(st % 4) + 16 kq rows + 256 (st / 4).
    constexpr int KBS = G::KSTEPS < 4 ? G::KSTEPS : 4;
    int koff[KBS];
#pragma unroll
    for (int j = 0; j < KBS; ++j)
        koff[j] = n * G::ROWL + 16 * ((4 * j + kb) ^ swz(n));
    // V reads (ds_read_b64_tr_b16): lane group kb reads keys
    // 32 ks + 16 hh + 4 kb + s/4 (s = lane in group), columns
    // 16 jb + 4 (s % 4) .. +3.  swz() of those keys is fixed per lane, so a
    // read = base(jb % 8) + (32 ks + 16 hh) rows + 256 (jb / 8).
    constexpr int VBS = G::DBLK < 8 ? G::DBLK : 8;
    int voff[VBS];
    {
        const int vkey = 4 * kb + (n >> 2);
        const int sw = swz(vkey);
#pragma unroll
        for (int j = 0; j < VBS; ++j)
            voff[j] = vkey * G::ROWL + 16 * ((2 * j + ((n & 3) >> 1)) ^ sw) + (n & 1) * 8;
    }

    Staged<D> stg;
    int rawn[4];  // block-table entries of the next tile to load
    char* buf0 = smem0;
    if constexpr (FP8) {
        stage_load<D>(stg, b, kp, vp, a.k_scale, a.v_scale, 0, tid, &bad);
        stage_store<D>(stg, buf0, buf0 + G::TILEB, (float*)(buf0 + 2 * G::TILEB), tid);
    } else {
        int raw0[4];
        fetch_pages(b, 0, raw0);
        issue_direct<D>(buf0, buf0 + G::TILEB, b, kp, vp, 0, wave, loff, raw0, &bad);
        fetch_pages(b, kKT, rawn);
        __builtin_amdgcn_s_waitcnt(0);
    }
    __syncthreads();

    auto tile_body = [&](int t, char* cbuf, char* nbuf) {
        const int tile0 = t * kKT;
        if (t + 1 < nt) {
            if constexpr (FP8)
                stage_load<D>(stg, b, kp, vp, a.k_scale, a.v_scale, tile0 + kKT, tid, &bad);
            else {
                issue_direct<D>(nbuf, nbuf + G::TILEB, b, kp, vp, tile0 + kKT, wave, loff, rawn,
                                &bad);
                fetch_pages(b, tile0 + 2 * kKT, rawn);
            }
        }
        const char* buf = cbuf;
        const char* ks = buf;
        const char* vs = buf + G::TILEB;
        const float* sc = (const float*)(buf + 2 * G::TILEB);
        const bool diag = tile0 + kKT - 1 > minpos;  // the causal edge crosses this tile

        // Two 32-key halves; per half: S^T (2 key blocks), a rescale check
        // (rarely taken), exp/sum/pack, PV (one 32-key k-step per d block).
        f32x4 acc[4];
        u32x4 pb2[2];  // P^T operands of the two 32-key k-steps
        // Operands of a 16-key block are read from LDS in one batch before its
        // MFMAs, so the reads' latency overlaps instead of gating each MFMA.
        auto s_half = [&](int hf) {
#pragma unroll
            for (int kq = 2 * hf; kq < 2 * hf + 2; ++kq) {
                u32x4 kw[G::KSTEPS];
#pragma unroll
                for (int st = 0; st < G::KSTEPS; ++st)
                    kw[st] = *(const u32x4*)(ks + koff[st % KBS] + kq * 16 * G::ROWL +
                                             256 * (st / KBS));
                acc[kq] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int st = 0; st < G::KSTEPS; ++st)
                    acc[kq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, kw[st]), __builtin_bit_cast(bf16x8, qop[st]),
                        acc[kq], 0, 0, 0);
            }
        };
        // One max check over the whole tile, before any of its scores is
        // turned into a probability: a rescale between the two halves would
        // leave the first half's P relative to the old max.
        auto check_tile = [&]() {
            float tmax = neg_inf();
#pragma unroll
            for (int kq = 0; kq < 4; ++kq) {
                const float s = FP8 ? sc[kq] * sm_log2 : sm_log2;
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    float v = acc[kq][x] * s;
                    if (diag && tile0 + 16 * kq + 4 * kb + x > pos)
                        v = neg_inf();
                    acc[kq][x] = v;
                    tmax = fmaxf(tmax, v);
                }
            }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
            if (__builtin_amdgcn_ballot_w64(tmax > m + kTau)) {
                const float mnew = fmaxf(m, tmax);
                const float alpha =
                    m == neg_inf() ? 0.f : (m == mnew ? 1.f : __builtin_amdgcn_exp2f(m - mnew));
                l = l * alpha;
#pragma unroll
                for (int jb = 0; jb < G::DBLK; ++jb)
                    O[jb] = O[jb] * alpha;
                m = mnew;
            }
        };
        auto softmax_half = [&](int hf) {
            const float muse = m == neg_inf() ? 0.f : m;
            float e[2][4];
            float psum = 0.f;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int kq = 2 * hf + j;
                const float vscale = FP8 ? sc[4 + kq] : 1.f;
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const float pe = __builtin_amdgcn_exp2f(acc[kq][x] - muse);
                    psum = psum + pe;
                    e[j][x] = FP8 ? pe * vscale : pe;
                }
            }
            pb2[hf][0] = pack_bf16(e[0][0], e[0][1]);
            pb2[hf][1] = pack_bf16(e[0][2], e[0][3]);
            pb2[hf][2] = pack_bf16(e[1][0], e[1][1]);
            pb2[hf][3] = pack_bf16(e[1][2], e[1][3]);
            psum = psum + __shfl_xor(psum, 16, 64);
            psum = psum + __shfl_xor(psum, 32, 64);
            l = l + psum;
        };
        auto pv_half = [&](int hf) {
            constexpr int NB = 8;  // d blocks per batch of V reads
#pragma unroll
            for (int j0 = 0; j0 < G::DBLK; j0 += NB) {
                u32x4 va[NB];
#pragma unroll
                for (int jj = 0; jj < NB; ++jj) {
                    const int jb = j0 + jj;
                    const char* v0 = vs + voff[jb % VBS] + 32 * hf * G::ROWL + 256 * (jb / VBS);
                    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS s16x4*)v0);
                    const s16x4 hi =
                        __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS s16x4*)(v0 + 16 * G::ROWL));
                    const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
                    const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
                    va[jj] = u32x4{l2[0], l2[1], h2[0], h2[1]};
                }
#pragma unroll
                for (int jj = 0; jj < NB; ++jj)
                    O[j0 + jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, va[jj]), __builtin_bit_cast(bf16x8, pb2[hf]),
                        O[j0 + jj], 0, 0, 0);
            }
        };
        s_half(0);
        s_half(1);
        check_tile();
        softmax_half(0);
        pv_half(0);
        softmax_half(1);
        pv_half(1);

        if (t + 1 < nt) {
            if constexpr (FP8)
                stage_store<D>(stg, nbuf, nbuf + G::TILEB, (float*)(nbuf + 2 * G::TILEB), tid);
            else
                __builtin_amdgcn_s_waitcnt(0);
        }
        __syncthreads();
    };
    for (int t = 0; t < nt; t += 2) {
        tile_body(t, smem0, smem1);
        if (t + 1 < nt)
            tile_body(t + 1, smem1, smem0);
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
    for (int jb = 0; jb < G::DBLK; ++jb) {
        const int d = 16 * jb + 4 * kb;
        u32x2 o;
        o[0] = nan ? 0x7FC07FC0u : pack_bf16(O[jb][0] * inv, O[jb][1] * inv);
        o[1] = nan ? 0x7FC07FC0u : pack_bf16(O[jb][2] * inv, O[jb][3] * inv);
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
    hipLaunchKernelGGL((prefill_kernel<D, FP8>), dim3(grid), dim3(kThreads), 0, stream, a);
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
