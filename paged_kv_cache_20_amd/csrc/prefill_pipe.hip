// prefill_pipe.hip -- the prefill chunk on a bf16 cache, with the work of
// each 32-row group split between two waves.
//
// Call shape: "kern manifest v7" schema, $defs.Batch (one sequence, as many
// rows as the chunk; `context` is the cached rows the call expands over).
// Row r of an n_rows chunk sits at position ctx_len - n_rows + r and attends
// to keys 0 .. that position (the window and floor, when given, raise the
// first key).
//
// Work decomposition (gfx950)
//   A workgroup of 8 waves owns one kv head and 128 query rows: 128 / g
//   consecutive positions x the g query heads sharing the kv head.  The rows
//   form 4 groups of 32 (two 16-row MFMA tiles).  Each group is served by a
//   pair of waves, one of each role:
//     score wave s (0..3)       S^T = K . Q^T for the group's 32 rows on
//                               v_mfma_f32_16x16x32_bf16 (Q^T in registers,
//                               K rows from LDS), the online softmax, and the
//                               probabilities P^T (bf16) written to LDS in the
//                               exact register layout of the PV operand
//     output wave 4 + s         O^T += V^T . P^T for the same rows (V^T read
//                               from LDS with the transposing reads, P^T read
//                               back from LDS), rescaled when the score wave
//                               raised a row's running maximum
//   Each wave reads every K (or V) operand once and feeds it to two matrix
//   instructions, one per 16-row tile, so the LDS bytes per flop are half of
//   a one-tile-per-wave kernel's; and each SIMD hosts one wave of each role,
//   so one wave's softmax or LDS latency overlaps the other's matrix work.
//   Roles run one tile apart: in iteration i the score waves turn tile i's
//   scores into probabilities while the output waves accumulate tile i - 1;
//   one barrier per iteration hands P, the rescale factors and the freshly
//   loaded tiles over.  The score waves are software-pipelined themselves:
//   the scores of tile i + 1 are computed on the matrix unit while tile i's
//   exponentials run.
//
// Tiles and buffers
//   Keys stream in 32-key tiles (two 16-token pages).  In iteration i the
//   score waves read K(i + 1) and load K(i + 2) into the buffer K(i) left
//   free; the output waves read V(i - 1) and load V(i); P and the rescale
//   factors of tiles i - 1 and i sit in two more buffers.  Each wave loads 8
//   key rows of one page per tile, by buffer loads that write LDS
//   directly.  The buffer descriptor of each page covers only its rows below
//   ctx_len, so rows past the context arrive as zeros; a block-table entry
//   outside the pool is never dereferenced and turns the workgroup's rows to
//   NaN.  Pages wholly below the first key any row attends are not read.
//   K and V rows are stored row-major (bf16), each row's 16-byte chunks
//   XOR-swizzled by the row index, so the operand reads of a column of rows
//   are conflict-free.
//
// Softmax
//   A row's 8 scores of a tile sit in the 4 lanes n, n + 16, n + 32, n + 48
//   of its score wave.  Each lane keeps its own part of the row sum; the row
//   maximum is gathered over the 4 lanes only when some lane's score exceeds
//   the running maximum by more than 2^8 (checked once per tile, before any
//   score of the tile becomes a probability).  The output wave then scales
//   its rows of O by the factor the score wave wrote.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

#define LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kKT = 32;      // keys per tile
constexpr int kRT = 2;       // 16-row MFMA tiles per wave
constexpr int kGroups = 4;   // 32-row groups per workgroup (score waves)
constexpr float kTau = 8.f;  // lazy-rescale threshold (log2 units)
constexpr int kRsrcFlags = 0x00020000;

__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }

// Two floats to a bf16 pair (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Physical 16-byte chunk of logical chunk c in LDS row r is c ^ swz(r).
// swz depends on r's low four bits only and is one-to-one on them; it keeps
// the K operand reads (one chunk of each of 16 consecutive rows) and the
// transposing V reads (4 rows per 16 lanes, two chunks) free of bank
// conflicts.
__device__ __forceinline__ int swz(int r)
{
    return ((r >> 2) & 1) | ((r & 1) << 1) | (((r >> 1) & 1) << 2) |
           ((((r >> 2) ^ (r >> 3)) & 1) << 3);
}

__device__ __forceinline__ float row_max4(float v)
{
    v = fmaxf(v, __shfl_xor(v, 16, 64));
    return fmaxf(v, __shfl_xor(v, 32, 64));
}

__device__ __forceinline__ float row_sum4(float v)
{
    v = v + __shfl_xor(v, 16, 64);
    return v + __shfl_xor(v, 32, 64);
}

template <int D>
struct PGeo {
    static constexpr int ROWL = 2 * D;              // bytes of one key row (pool and LDS)
    static constexpr int TILEB = kKT * ROWL;        // one K (or V) tile in LDS
    static constexpr int KSTEPS = D / 32;           // k-steps of QK^T
    static constexpr int DBLK = D / 16;             // 16-wide d blocks of O^T
    static constexpr int ROWS = 16 * kRT * kGroups; // query rows per workgroup
    static constexpr int CPRL = ROWL / 16;          // 16-byte chunks per row
    static constexpr int RPI = 1024 / ROWL;         // key rows per LDS-direct load
    static constexpr int LROWS = kKT / 4;           // key rows a wave loads per tile
    static constexpr int LINS = LROWS / RPI;        // loads per wave per tile
    static_assert(LINS * RPI == LROWS, "a wave's rows fill whole loads");
};

// A loop phase known at compile time (the tile index mod 3 selects the K and
// V slots, so each slot is its own LDS array and the compiler can tell the
// tile loads in flight from the reads of another slot).
template <int N>
struct Ph {
    static constexpr int v = N;
};

// Shared state of one workgroup besides the K and V slots.
template <int D>
struct Smem {
    u32x4 p[2][kGroups][kRT][64];      // P^T operands, by (tile parity, group, row tile, lane)
    float alpha[2][kGroups][kRT][16];  // rescale factor of each row
    int flag[2][kGroups];              // a group raised some row's maximum in that tile
    float lsum[kGroups][kRT][16];      // row sums at the end
    int bad;
};

struct Seq {
    int C;     // keys in the sequence (ctx_len)
    int kend;  // keys the workgroup loads: min(C, its tiles' end)
    int lo;    // first key any row of the workgroup attends (window / floor)
    int kh, Hk;
    int64_t n_pages;
    __amdgpu_buffer_rsrc_t rbt;  // the sequence's block-table row, ceil(kend / 16) entries
};

// Block-table entry of the page holding key0 .. key0 + 15 (0 past the
// workgroup's pages; load_rows decides whether the page is read).  Always one
// bounds-checked load, so every iteration issues the same number of loads;
// nothing here consumes the value, so its wait comes at its use.
__device__ __forceinline__ int fetch_page(const Seq& b, int key0)
{
    return (int)__builtin_amdgcn_raw_buffer_load_b32(b.rbt, (uint32_t)(key0 >> 4) * 4u, 0, 0);
}

// This wave's 8 key rows of one tensor's tile (one page), copied to LDS by
// buffer loads that write LDS directly.  key0: the page's first key; prow:
// the wave's first row in the page (0 or 8); dst: the page's first row in
// the tile's LDS buffer.  A page the workgroup does not read gets a
// descriptor of no rows: the loads are still issued (zeros), so the count
// per iteration is fixed.
template <int D>
__device__ __forceinline__ void load_rows(char* dst, const uint8_t* pool, const Seq& b, int key0,
                                          int prow, int raw, const int (&loff)[PGeo<D>::LINS],
                                          int* bad)
{
    using G = PGeo<D>;
    const int p = __builtin_amdgcn_readfirstlane(raw);
    int pg = 0, rows = 0;
    if (key0 < b.kend && key0 + 16 > b.lo) {
        if (p < 0 || (int64_t)p >= b.n_pages) {
            *bad = 1;
        } else {
            pg = p;
            rows = min(16, b.C - key0);
        }
    }
    const int64_t base = ((int64_t)pg * b.Hk + b.kh) * 16 * G::ROWL;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(pool + base), (short)0, rows * G::ROWL,
                                          kRsrcFlags);
#pragma unroll
    for (int i = 0; i < G::LINS; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (LDS void*)(dst + (prow + i * G::RPI) * G::ROWL), 16, loff[i], 0, 0, 0);
}

// The per-tile barrier.  Every LDS access of this wave is complete
// (lgkmcnt 0) and all but its N newest vector-memory loads (the tile loads
// just issued, which write LDS directly) have landed; then s_barrier.
// __syncthreads() would wait for every load that writes LDS, which would
// leave each tile load one iteration instead of two.  The empty asm
// statements keep the compiler from moving memory accesses across.  (gfx9
// s_waitcnt encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8.)
template <int N>
__device__ __forceinline__ void tile_barrier()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

template <int D>
__global__ __launch_bounds__(512, 2) void prefill_pipe_kernel(PrefillArgs a)
{
    using G = PGeo<D>;
    // K and V of tiles t = 0, 1, 2 (mod 3), then the rest.
    __shared__ __attribute__((aligned(1024))) char s_k0[G::TILEB];
    __shared__ __attribute__((aligned(1024))) char s_k1[G::TILEB];
    __shared__ __attribute__((aligned(1024))) char s_k2[G::TILEB];
    __shared__ __attribute__((aligned(1024))) char s_v0[G::TILEB];
    __shared__ __attribute__((aligned(1024))) char s_v1[G::TILEB];
    __shared__ __attribute__((aligned(1024))) char s_v2[G::TILEB];
    __shared__ __attribute__((aligned(1024))) Smem<D> sm;
    auto kslot = [&](auto ph) -> char* {
        constexpr int P = decltype(ph)::v % 3;
        return P == 0 ? s_k0 : P == 1 ? s_k1 : s_k2;
    };
    auto vslot = [&](auto ph) -> char* {
        constexpr int P = decltype(ph)::v % 3;
        return P == 0 ? s_v0 : P == 1 ? s_v1 : s_v2;
    };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, kb = lane >> 4;
    const int Hk = a.n_head_kv, H = a.n_head, g = H / Hk, BP = G::ROWS / g;
    int n_rows = a.n_rows, ctx_len = a.ctx_len;
    int64_t tok0 = 0;
    const int32_t* bt = a.block_table;
    const int npbm = ((a.cu_seqlens ? a.max_q_len : a.n_rows) + BP - 1) / BP;
    const int nblk = (a.cu_seqlens ? a.n_var : 1) * npbm * Hk;
    // XCD-aware placement: consecutive list entries (same sequence and kv
    // head) go to the same XCD; heavier (later) position blocks first.
    const int per_xcd = (nblk + 7) / 8;
    const int L = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (L >= nblk)
        return;
    const int sv = L / (npbm * Hk);
    const int rem = L - sv * (npbm * Hk);
    if (a.cu_seqlens) {
        const int c0 = a.cu_seqlens[sv], c1 = a.cu_seqlens[sv + 1];
        ctx_len = a.ctx_lens[sv];
        n_rows = c1 - c0;
        if (c0 < 0 || c1 > a.n_tok || n_rows < 1 || n_rows > a.max_q_len || ctx_len < n_rows ||
            (int64_t)ctx_len > (int64_t)a.max_pages * 16)
            return;
        tok0 = c0;
        bt = a.block_table + (int64_t)sv * a.max_pages;
    }
    const int npb = (n_rows + BP - 1) / BP;
    const int kh = rem / npbm;
    const int pbi = rem - kh * npbm;
    if (pbi >= npb)
        return;
    const int pb = npb - 1 - pbi;

    const int base_pos = ctx_len - n_rows;
    const int rlast = min(n_rows, (pb + 1) * BP) - 1;
    const int maxpos = base_pos + rlast;  // last key any row here needs
    const int minpos = base_pos + pb * BP;
    const int nt = (maxpos + kKT) / kKT;
    auto key_floor = [&](int p) { return max(a.kv_floor, a.window > 0 ? p - a.window + 1 : 0); };
    const int lo_min = key_floor(minpos), lo_max = key_floor(maxpos);
    const int ts = lo_min / kKT;  // first tile with a key to attend
    const int T = nt - ts;        // tiles

    Seq b;
    b.C = ctx_len;
    b.kend = min(ctx_len, nt * kKT);
    b.lo = lo_min;
    b.kh = kh;
    b.Hk = Hk;
    b.n_pages = a.n_pages;
    b.rbt = __builtin_amdgcn_make_buffer_rsrc((void*)bt, (short)0,
                                              (int)(((b.kend + 15) >> 4) * 4), kRsrcFlags);

    // The group's rows: wave grp's lane n, row tile rt holds workgroup row
    // 16 (2 grp + rt) + n.
    const int grp = wave & 3;
    int row[kRT], head[kRT], pos[kRT], klo[kRT];
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
        const int wrow = 16 * (kRT * grp + rt) + n;
        const int hg = wrow / BP, p = wrow - hg * BP;
        row[rt] = pb * BP + p;
        head[rt] = kh * g + hg;
        pos[rt] = row[rt] < n_rows ? base_pos + row[rt] : -1;
        klo[rt] = key_floor(pos[rt]);
    }

    if (tid == 0)
        sm.bad = 0;
    int bad = 0;
    const uint8_t* kp = (const uint8_t*)a.k_pool;
    const uint8_t* vp = (const uint8_t*)a.v_pool;

    // Loads: wave w fills key rows 8 (w & 1) .. + 7 of page (w >> 1) & 1 of
    // every tile of its tensor (K for the score waves, V for the output
    // waves).  Instruction i writes LDS rows prow + i RPI .. + RPI - 1 of the
    // page linearly; lane l of it fetches logical chunk pc ^ swz(row) of row
    // rr, so the tile ends up swizzled.  Each wave issues one table load and
    // then G::LINS tile loads per iteration, so "all but this iteration's
    // tile loads done" is vmcnt <= G::LINS.
    const int lpage = (wave >> 1) & 1, prow = 8 * (wave & 1);
    const int pr0 = 16 * lpage;  // the wave's page's first row in a tile
    int loff[G::LINS];
    {
        const int rr = lane / G::CPRL, pc = lane % G::CPRL;
#pragma unroll
        for (int i = 0; i < G::LINS; ++i) {
            const int r = prow + i * G::RPI + rr;  // row in the page
            loff[i] = r * G::ROWL + ((pc ^ swz(r)) * 16);
        }
    }
    constexpr int kInFlight = G::LINS;

    // Prologue: K(0..2) (score waves) and V(0) (output waves), and the table
    // entry of the next tile each role loads (K(3), V(1)), all landed.
    const int k0 = ts * kKT + pr0;  // the wave's page's first key in tile ts
    const bool score = wave < 4;
    int raw_next;
    if (score) {
        load_rows<D>(s_k0 + pr0 * G::ROWL, kp, b, k0, prow, fetch_page(b, k0), loff, &bad);
        load_rows<D>(s_k1 + pr0 * G::ROWL, kp, b, k0 + kKT, prow, fetch_page(b, k0 + kKT), loff,
                     &bad);
        load_rows<D>(s_k2 + pr0 * G::ROWL, kp, b, k0 + 2 * kKT, prow,
                     fetch_page(b, k0 + 2 * kKT), loff, &bad);
        raw_next = fetch_page(b, k0 + 3 * kKT);
    } else {
        load_rows<D>(s_v0 + pr0 * G::ROWL, vp, b, k0, prow, fetch_page(b, k0), loff, &bad);
        raw_next = fetch_page(b, k0 + kKT);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    if (score) {
        // ---- score wave: Q^T in registers, K from LDS, softmax, P^T out.
        u32x4 qop[kRT][G::KSTEPS];  // Q^T operand: d = 32 st + 8 kb + 0..7
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
            const bool valid = row[rt] < n_rows;
            const uint16_t* q =
                (const uint16_t*)a.q + ((tok0 + (valid ? row[rt] : 0)) * H + head[rt]) * D;
#pragma unroll
            for (int st = 0; st < G::KSTEPS; ++st)
                qop[rt][st] = valid ? *(const u32x4*)(q + 32 * st + 8 * kb) : u32x4{0u, 0u, 0u, 0u};
        }
        constexpr int KBS = G::KSTEPS < 4 ? G::KSTEPS : 4;
        int koff[KBS];
#pragma unroll
        for (int j = 0; j < KBS; ++j)
            koff[j] = n * G::ROWL + 16 * ((4 * j + kb) ^ swz(n));
        const float sm_log2 = kLog2e / __builtin_sqrtf((float)D);
        float m[kRT], l[kRT];
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
            m[rt] = neg_inf();
            l[rt] = 0.f;
        }
        // S^T[key][row] of a tile's two 16-key blocks, K rows from buffer ks.
        auto scores = [&](const char* ks, f32x4 (&s)[kRT][2]) {
#pragma unroll
            for (int kq = 0; kq < 2; ++kq) {
                u32x4 kw[G::KSTEPS];
#pragma unroll
                for (int st = 0; st < G::KSTEPS; ++st)
                    kw[st] = *(const u32x4*)(ks + koff[st % KBS] + kq * 16 * G::ROWL +
                                             256 * (st / KBS));
#pragma unroll
                for (int rt = 0; rt < kRT; ++rt) {
                    s[rt][kq] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int st = 0; st < G::KSTEPS; ++st)
                        s[rt][kq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, kw[st]),
                            __builtin_bit_cast(bf16x8, qop[rt][st]), s[rt][kq], 0, 0, 0);
                }
            }
        };
        // Software pipeline: iteration i computes the scores of tile i + 1
        // on the matrix unit while tile i's exponentials run (s holds tile i).
        f32x4 s[kRT][2];
        scores(s_k0, s);
        // Iteration 0 loads K(3) into K(0)'s slot: every score wave must have
        // read K(0) first (the output waves take this barrier before their
        // loop).
        __syncthreads();
        int rawk = raw_next;  // K(3)'s page
        // Iteration i, phase P = i mod 3.
        auto body = [&](int i, auto ph) {
            constexpr int P = decltype(ph)::v;
            // K(i + 3) into the slot K(i) held (read last in iteration i - 1);
            // its table entry was fetched before K(i + 2)'s loads were issued,
            // so waiting for it does not wait for them.
            const int rawn = fetch_page(b, k0 + (i + 4) * kKT);
            load_rows<D>(kslot(Ph<P>()) + pr0 * G::ROWL, kp, b, k0 + (i + 3) * kKT, prow, rawk,
                         loff, &bad);
            rawk = rawn;
            if (i < T) {
                const int buf = i & 1;
                const int tile0 = (ts + i) * kKT;
                // Scale (log2 units); on a tile crossing the causal edge or a
                // row's first key, mask.  Then the lane-local max check.
                const bool diag = tile0 + kKT - 1 > minpos || tile0 < lo_max;
                float sx = sm_log2;
                float lmax[kRT];
                if (diag) {
#pragma unroll
                    for (int rt = 0; rt < kRT; ++rt) {
                        float mx = neg_inf();
#pragma unroll
                        for (int kq = 0; kq < 2; ++kq)
#pragma unroll
                            for (int x = 0; x < 4; ++x) {
                                const int key = tile0 + 16 * kq + 4 * kb + x;
                                const float v = key > pos[rt] || key < klo[rt]
                                                    ? neg_inf()
                                                    : s[rt][kq][x] * sm_log2;
                                s[rt][kq][x] = v;
                                mx = fmaxf(mx, v);
                            }
                        lmax[rt] = mx;
                    }
                    sx = 1.f;
                } else {
#pragma unroll
                    for (int rt = 0; rt < kRT; ++rt) {
                        float mx = neg_inf();
#pragma unroll
                        for (int kq = 0; kq < 2; ++kq)
                            mx = fmaxf(mx, fmaxf(fmaxf(s[rt][kq][0], s[rt][kq][1]),
                                                 fmaxf(s[rt][kq][2], s[rt][kq][3])));
                        lmax[rt] = mx * sm_log2;
                    }
                }
                bool up = false;
#pragma unroll
                for (int rt = 0; rt < kRT; ++rt)
                    up = up || lmax[rt] > m[rt] + kTau;
                const bool any = __builtin_amdgcn_ballot_w64(up) != 0;
                if (any) {
#pragma unroll
                    for (int rt = 0; rt < kRT; ++rt) {
                        const float mnew = fmaxf(m[rt], row_max4(lmax[rt]));
                        const float alpha =
                            m[rt] == neg_inf() ? 0.f : __builtin_amdgcn_exp2f(m[rt] - mnew);
                        l[rt] = l[rt] * alpha;
                        m[rt] = mnew;
                        if (kb == 0)
                            sm.alpha[buf][grp][rt][n] = alpha;
                    }
                }
                if (lane == 0)
                    sm.flag[buf][grp] = any ? 1 : 0;

                // The scores of tile i + 1 (stale K past the last tile: never
                // used), issued beside tile i's probabilities, this lane's part
                // of the row sums, and the P^T operand: k index j of the 32-key
                // step is key 16 (j / 4) + 4 kb + j % 4, matching the V^T reads.
                f32x4 sn[kRT][2];
                scores(kslot(Ph<P + 1>()), sn);
#pragma unroll
                for (int rt = 0; rt < kRT; ++rt) {
                    const float mu = m[rt] == neg_inf() ? 0.f : m[rt];
                    float e[2][4];
#pragma unroll
                    for (int kq = 0; kq < 2; ++kq)
#pragma unroll
                        for (int x = 0; x < 4; ++x)
                            e[kq][x] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rt][kq][x], sx, -mu));
                    l[rt] = l[rt] + (((e[0][0] + e[0][1]) + (e[0][2] + e[0][3])) +
                                     ((e[1][0] + e[1][1]) + (e[1][2] + e[1][3])));
                    u32x4 pw;
                    pw[0] = pack_bf16(e[0][0], e[0][1]);
                    pw[1] = pack_bf16(e[0][2], e[0][3]);
                    pw[2] = pack_bf16(e[1][0], e[1][1]);
                    pw[3] = pack_bf16(e[1][2], e[1][3]);
                    sm.p[buf][grp][rt][lane] = pw;
                }
#pragma unroll
                for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
                    for (int kq = 0; kq < 2; ++kq)
                        s[rt][kq] = sn[rt][kq];
            }
            // K(i + 2) (issued in iteration i - 1) has landed; K(i + 3) may
            // still be in flight.
            tile_barrier<kInFlight>();
        };
        for (int i = 0; i <= T; i += 3) {
            body(i, Ph<0>());
            if (i + 1 <= T)
                body(i + 1, Ph<1>());
            if (i + 2 <= T)
                body(i + 2, Ph<2>());
        }
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
            const float ls = row_sum4(l[rt]);
            if (kb == 0)
                sm.lsum[grp][rt][n] = ls;
        }
        if (bad)
            sm.bad = 1;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    } else {
        // ---- output wave: O^T += V^T . P^T, one tile behind.
        constexpr int VBS = G::DBLK < 8 ? G::DBLK : 8;
        int voff[VBS];
        {
            const int vkey = 4 * kb + (n >> 2);
            const int sw = swz(vkey);
#pragma unroll
            for (int j = 0; j < VBS; ++j)
                voff[j] = vkey * G::ROWL + 16 * ((2 * j + ((n & 3) >> 1)) ^ sw) + (n & 1) * 8;
        }
        f32x4 O[kRT][G::DBLK];
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
            for (int jb = 0; jb < G::DBLK; ++jb)
                O[rt][jb] = f32x4{0.f, 0.f, 0.f, 0.f};
        __syncthreads();  // the score waves' barrier after the tile-0 scores
        int rawv = raw_next;  // V(1)'s page
        // Iteration i, phase P = i mod 3: V(i + 1) goes to slot P + 1, V(i - 1)
        // is read from slot P + 2 (mod 3).
        auto body = [&](int i, auto ph) {
            constexpr int P = decltype(ph)::v;
            // V(i + 1) into the slot V(i - 2) held (read last in iteration
            // i - 1); table entries are fetched an iteration ahead, before the
            // previous tile's loads.
            const int rawn = fetch_page(b, k0 + (i + 2) * kKT);
            load_rows<D>(vslot(Ph<P + 1>()) + pr0 * G::ROWL, vp, b, k0 + (i + 1) * kKT, prow,
                         rawv, loff, &bad);
            rawv = rawn;
            if (i >= 1) {
                const int buf = (i - 1) & 1;
                if (sm.flag[buf][grp]) {
#pragma unroll
                    for (int rt = 0; rt < kRT; ++rt) {
                        const float al = sm.alpha[buf][grp][rt][n];
#pragma unroll
                        for (int jb = 0; jb < G::DBLK; ++jb)
                            O[rt][jb] = O[rt][jb] * al;
                    }
                }
                u32x4 pw[kRT];
#pragma unroll
                for (int rt = 0; rt < kRT; ++rt)
                    pw[rt] = sm.p[buf][grp][rt][lane];
                const char* vr = vslot(Ph<P + 2>());
#pragma unroll
                for (int jb = 0; jb < G::DBLK; ++jb) {
                    const char* v0 = vr + voff[jb % VBS] + 256 * (jb / VBS);
                    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS s16x4*)v0);
                    const s16x4 hi =
                        __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS s16x4*)(v0 + 16 * G::ROWL));
                    const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
                    const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
                    const u32x4 va = u32x4{l2[0], l2[1], h2[0], h2[1]};
#pragma unroll
                    for (int rt = 0; rt < kRT; ++rt)
                        O[rt][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, va), __builtin_bit_cast(bf16x8, pw[rt]),
                            O[rt][jb], 0, 0, 0);
                }
            }
            // V(i) (issued in iteration i - 1) has landed; V(i + 1) may still
            // be in flight.
            tile_barrier<kInFlight>();
        };
        for (int i = 0; i <= T; i += 3) {
            body(i, Ph<0>());
            if (i + 1 <= T)
                body(i + 1, Ph<1>());
            if (i + 2 <= T)
                body(i + 2, Ph<2>());
        }
        if (bad)
            sm.bad = 1;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        const bool nan = sm.bad != 0;
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
            if (row[rt] >= n_rows)
                continue;
            const float inv = 1.f / sm.lsum[grp][rt][n];
            uint16_t* out = (uint16_t*)a.out + ((tok0 + row[rt]) * H + head[rt]) * D;
#pragma unroll
            for (int jb = 0; jb < G::DBLK; ++jb) {
                const int d = 16 * jb + 4 * kb;
                u32x2 o;
                o[0] = nan ? 0x7FC07FC0u : pack_bf16(O[rt][jb][0] * inv, O[rt][jb][1] * inv);
                o[1] = nan ? 0x7FC07FC0u : pack_bf16(O[rt][jb][2] * inv, O[rt][jb][3] * inv);
                *(u32x2*)(out + d) = o;
            }
        }
    }
}

template <int D>
hipError_t launch_d(const PrefillArgs& a, hipStream_t stream)
{
    using G = PGeo<D>;
    const int g = a.n_head / a.n_head_kv;
    const int BP = G::ROWS / g;
    const int npbm = ((a.cu_seqlens ? a.max_q_len : a.n_rows) + BP - 1) / BP;
    const int64_t nblk = (int64_t)(a.cu_seqlens ? a.n_var : 1) * npbm * a.n_head_kv;
    if (nblk > (int64_t)1 << 30)
        return hipErrorInvalidValue;
    const int grid = (int)((nblk + 7) / 8) * 8;
    if (a.ev_start)
        (void)hipEventRecord(a.ev_start, stream);
    hipLaunchKernelGGL((prefill_pipe_kernel<D>), dim3(grid), dim3(512), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && a.ev_stop)
        (void)hipEventRecord(a.ev_stop, stream);
    return e;
}

}  // namespace

// bf16 cache, head_dim 128 or 256, g a divisor of 128; other shapes are
// refused (hipErrorNotSupported) and take the one-role kernel.
hipError_t launch_prefill_pipe(const PrefillArgs& a, hipStream_t stream)
{
    const int g = a.n_head / a.n_head_kv;
    if (a.fp8 || a.qk_fp8 || g > 128 || 128 % g != 0)
        return hipErrorNotSupported;
    if (a.head_dim == 128)
        return launch_d<128>(a, stream);
    if (a.head_dim == 256)
        return launch_d<256>(a, stream);
    return hipErrorNotSupported;
}

}  // namespace pa
