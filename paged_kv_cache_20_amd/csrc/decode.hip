// decode.hip -- split-K paged attention for the decode step (1 row per
// sequence) and the speculative verify round (8 rows per sequence), gfx950.
//
// Call shapes: "kern manifest v7" schema, $defs.Batch (rows 1 for a decode
// step, exactly 8 for a speculative round); row r of a call with R rows sits
// at position ctx_len - R + r ($defs.Fill "seq_len" counts the call's rows).
//
// Work decomposition
//   A work item is (sequence s, split j, kv head kh): keys [P j, P j + P) of
//   s, clipped to ctx_len, with P = 1024 for the fp8 cache at head_dim 128
//   and 512 otherwise.  Split boundaries are absolute multiples of P,
//   so the items a row takes part in, and everything computed inside them,
//   depend on the row's position and its sequence's own data only.  Items
//   are listed full splits first, then the partial last splits from the
//   longest; each wave of a persistent grid takes one item per round of the
//   list, rounds walked in alternating directions, so the waves' shares of
//   keys even out and the grid's last items are its shortest.  Which wave
//   takes an item changes nothing in its arithmetic.  The block-table
//   entries of a wave's next item are fetched while it works on the current
//   one.
//
// Streaming
//   Keys stream in tiles of KT (16 or 32, fixed per head_dim and KV dtype)
//   through a ring of NBUF register buffers: the loads of tile i + NBUF - 1
//   are issued before tile i is computed, so NBUF - 1 tiles are in flight
//   while one is consumed.  Every load is a bounds-checked buffer load whose
//   resource covers only the rows of its (page, kv head) chunk below the end
//   of the item: rows past the context, and whole pages past the item, read
//   as zeros without touching memory.  No load sits under a branch, so the
//   compiler's counter waits release each tile as soon as its own loads are
//   done.  Page ids and fp8 scales are wave-uniform (scalar registers).
//   bf16 at head_dim 256 with two slot tiles per item streams through two
//   LDS slots per wave instead (loads that write LDS, two tiles ahead; see
//   the LR form below).
//
// Inside an item (one 64-lane wave)
//   Query rows are packed into 16-slot MFMA tiles.  A tile holds floor(16/g)
//   positions x g heads of the kv group (g = n_head / n_head_kv); position p
//   and head-in-group c sit in slot g * (p mod floor(16/g)) + c, so a
//   position occupies the same MFMA column in a decode call and in a verify
//   call.  Per key tile:
//     S^T[key][slot] = K . Q^T     v_mfma_f32_16x16x32_bf16, keys as rows
//     online softmax per slot      exp2, max/sum across the wave's 4 k-groups
//     O[slot][d]    += P . V       v_mfma_f32_16x16x32_bf16 (32-key tiles) or
//                                  v_mfma_f32_16x16x16_bf16 (16-key tiles)
//   The S^T accumulator layout (lane = slot + 16 * key group) is exactly the
//   A-operand layout P needs, so P never moves between lanes.  K is read in
//   A-operand order (16-byte pieces, one key row per lane); V is read
//   row-contiguous (each 16 lanes cover whole token rows) and transposed in
//   registers with byte permutes.  fp8 codes become bf16 exactly in
//   registers; the K scale multiplies the scores, the V scale is folded into
//   P, both per page.  Keys past a row's position are masked; a fully masked
//   tile leaves m, l and O bit-identical.
//
// Combine: per (sequence, row, head), splits 0 .. floor(pos / P) are merged
// in a fixed order that depends on their count only: M = max m_j,
// w_j = exp2(m_j - M), den = sum w_j l_j (a fixed butterfly inside each group
// of 64 splits, groups in increasing order), num = sum w_j o_j (j
// increasing), out = num / den rounded to bf16.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;  // waves per block
constexpr float kLog2e = 1.4426950408889634f;
// Word 3 of a raw buffer resource on gfx9: 32-bit data format, no swizzle;
// accesses at or past num_records return zero.
constexpr int kRsrcFlags = 0x00020000;
// A buffer offset past every resource the kernels build (each covers less
// than 2 GiB), with room for the instruction offsets added to it.
constexpr uint32_t kFar = 0x80000000u;

__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }

__device__ __forceinline__ uint32_t bf16_bits(float x)
{
    __bf16 b = (__bf16)x;  // round to nearest even
    return (uint32_t)__builtin_bit_cast(uint16_t, b);
}

// Two floats to a bf16 pair (round to nearest even), one conversion.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Two e4m3 codes (bytes 2*hi, 2*hi+1 of w) -> two bf16, exact.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w)
{
    bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HI);
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

// The value of lane l ^ 16 (l ^ 32) at lane l, by gfx950's row-pair (half)
// swap, a VALU operation: no LDS round trip and no counter wait.  Each swap
// exchanges one operand's odd rows (upper half) with the other's even rows
// (lower half); with both operands x, lanes of the even rows (lower half)
// find their partner in the second result, the others in the first.
__device__ __forceinline__ float xor16_f(float v)
{
    const uint32_t x = __builtin_bit_cast(uint32_t, v);
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    const bool odd = (threadIdx.x >> 4) & 1;
    return __builtin_bit_cast(float, odd ? r[0] : r[1]);
}
__device__ __forceinline__ float xor32_f(float v)
{
    const uint32_t x = __builtin_bit_cast(uint32_t, v);
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    const bool upper = (threadIdx.x >> 5) & 1;
    return __builtin_bit_cast(float, upper ? r[0] : r[1]);
}

__device__ __forceinline__ int rdlane(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }
__device__ __forceinline__ float rdlane_f(float v, int lane)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             kRsrcFlags);
}

template <int D, bool FP8>
struct Geo {
    static constexpr int EB = FP8 ? 1 : 2;      // bytes per stored element
    static constexpr int ROWB = D * EB;         // bytes per token row of one kv head
    static constexpr int CHUNKB = 16 * ROWB;    // bytes of one (page, kv head) chunk
    static constexpr int STEPS = D / 32;        // k-steps of the QK^T contraction
    static constexpr int KLD = ROWB / 64;       // 16-byte K loads per lane per 16-key block
    static constexpr int VPB = ROWB / 16;       // V bytes per lane per token
    static constexpr int VDW = VPB / 4;         // ... in dwords
    static constexpr int DB = D / 16;           // output columns per lane (d blocks)
    // Keys per tile: 32, except bf16 at head_dim 256 (16, one page), which
    // keeps a tile at 16 KiB.  A property of (head_dim, dtype) only, so a
    // row's arithmetic never depends on how many rows the call has.
    static constexpr int KT = (!FP8 && D == 256) ? 16 : 32;
    // Keys per split (see decode_chunk); likewise fixed per (head_dim, dtype).
    static constexpr int CHUNK = (D == 128 && FP8) ? 1024 : 512;
    // A lane holds one block-table entry of an item: at most 64 pages.
    static_assert(CHUNK / 16 <= 64, "a split spans at most 64 pages");
    static constexpr int KB = KT / 16;          // 16-key blocks per tile
    static constexpr int KEYS = 4 * KB;         // keys a lane feeds to the PV product
};

template <int D, bool FP8>
struct Raw {
    u32x4 k[Geo<D, FP8>::KB][Geo<D, FP8>::KLD];
    uint32_t v[Geo<D, FP8>::KEYS][Geo<D, FP8>::VDW];
};

// Register plan of an instantiation: waves per SIMD it is compiled for
// (two where two tiles, Q and O fit in half the register file) and the depth
// of its tile ring.  Items are padded to a multiple of the depth; padding
// tiles load nothing, so p of them at an item's end leave the ring NBUF - 1 - p
// real tiles ahead of the item's last tile.  Depth 4 (no padding for a full
// item of 16 or 32 tiles) where four tiles fit beside Q and O; with one wave
// per SIMD, depth 3 where a full item has 32 tiles (one padding tile); else
// depth 2 (no padding).  With one wave per SIMD the O accumulators live in
// the AGPR half of the file.
template <int D, bool FP8, int NT>
struct Plan {
    using G = Geo<D, FP8>;
    static constexpr int RAW = G::KB * G::KLD * 4 + G::KEYS * G::VDW;  // dwords per tile
    static constexpr int QOP = NT * G::STEPS * 4;
    static constexpr int OREG = NT * G::DB * 4;
    static constexpr int ITEM_TILES = G::CHUNK / G::KT;
    static constexpr int OCC = (2 * RAW + QOP + OREG <= 176) ? 2 : 1;
    static constexpr int NBUF =
        OCC == 2 ? ((4 * RAW + 2 * QOP + OREG <= 192) ? 4 : 2)
                 : ((ITEM_TILES % 3 == 2 && 3 * RAW + QOP <= 224) ? 3 : 2);
    // Whether the next item's query operands are loaded into a second set of
    // registers during the current item's last tiles (one slot tile only;
    // larger calls load them after the current item's last tile).
    static constexpr bool PREQ = NT == 1;
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

// Loads of one key tile.  pg0/pg1: pages of its two 16-key blocks (pg1 is
// unused for 16-key tiles); n0/n1: rows of each page inside the item (0..16).
// koff: this lane's byte offset of its K row piece, voff: of its first V row
// piece, inside a chunk.  Key kk = 4 kb + i (i < 4) or 16 + 4 kb + (i - 4)
// of the tile feeds PV k-slot i of lane group kb; those are the keys the
// lane's S^T accumulators hold.
template <int D, bool FP8>
__device__ __forceinline__ void load_tile(Raw<D, FP8>& t, const uint8_t* kp, const uint8_t* vp,
                                          int64_t chunk0, int64_t chunk1, int n0, int n1,
                                          uint32_t koff, uint32_t voff)
{
    using G = Geo<D, FP8>;
#pragma unroll
    for (int kblk = 0; kblk < G::KB; ++kblk) {
        const int64_t ch = kblk ? chunk1 : chunk0;
        const int nr = kblk ? n1 : n0;
        const __amdgpu_buffer_rsrc_t rk = rsrc(kp + ch * G::CHUNKB, (uint32_t)(nr * G::ROWB));
#pragma unroll
        for (int c = 0; c < G::KLD; ++c)
            t.k[kblk][c] = __builtin_amdgcn_raw_buffer_load_b128(rk, koff + 64 * c, 0, 0);
    }
#pragma unroll
    for (int kblk = 0; kblk < G::KB; ++kblk) {
        const int64_t ch = kblk ? chunk1 : chunk0;
        const int nr = kblk ? n1 : n0;
        const __amdgpu_buffer_rsrc_t rv = rsrc(vp + ch * G::CHUNKB, (uint32_t)(nr * G::ROWB));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t off = voff + i * G::ROWB;
            uint32_t* dst = t.v[4 * kblk + i];
            if constexpr (G::VDW == 2) {
                const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(rv, off, 0, 0);
                dst[0] = w[0];
                dst[1] = w[1];
            } else {
#pragma unroll
                for (int c = 0; c < G::VDW / 4; ++c) {
                    const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(rv, off + 16 * c, 0, 0);
                    dst[4 * c + 0] = w[0];
                    dst[4 * c + 1] = w[1];
                    dst[4 * c + 2] = w[2];
                    dst[4 * c + 3] = w[3];
                }
            }
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

template <int D, bool FP8, int NT, bool WIN, bool ILP>
__device__ __forceinline__ void compute_tile(const Raw<D, FP8>& t, const u32x4 (&qop)[NT][D / 32],
                                             const int (&first)[NT], const int (&last)[NT],
                                             float (&m)[NT], float (&l)[NT],
                                             f32x4 (&O)[NT][D / 16], int kt, float sc0, float sc1,
                                             float vs0, float vs1, int kb)
{
    using G = Geo<D, FP8>;
    constexpr int KB = G::KB;
    f32x4 acc[KB][NT];
#pragma unroll
    for (int kblk = 0; kblk < KB; ++kblk)
#pragma unroll
        for (int tau = 0; tau < NT; ++tau)
            acc[kblk][tau] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < G::STEPS; ++st) {
#pragma unroll
        for (int kblk = 0; kblk < KB; ++kblk) {
            const bf16x8 ka = k_operand<D, FP8>(t.k[kblk], st);
#pragma unroll
            for (int tau = 0; tau < NT; ++tau)
                acc[kblk][tau] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    ka, __builtin_bit_cast(bf16x8, qop[tau][st]), acc[kblk][tau], 0, 0, 0);
        }
    }

    uint32_t pa[NT][2 * KB];
    float alpha[NT];
#pragma unroll
    for (int tau = 0; tau < NT; ++tau) {
        float sv[KB][4];
        float tmax = neg_inf();
#pragma unroll
        for (int kblk = 0; kblk < KB; ++kblk)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = kt + 16 * kblk + 4 * kb + r;
                const float x = acc[kblk][tau][r] * (kblk ? sc1 : sc0);
                // (without a window or floor every first[] is 0: one compare)
                const bool in = WIN ? key <= last[tau] && key >= first[tau] : key <= last[tau];
                sv[kblk][r] = in ? x : neg_inf();
                tmax = fmaxf(tmax, sv[kblk][r]);
            }
        tmax = fmaxf(tmax, xor16_f(tmax));
        tmax = fmaxf(tmax, xor32_f(tmax));
        const float mnew = fmaxf(m[tau], tmax);
        const float muse = mnew == neg_inf() ? 0.f : mnew;
        const float al = m[tau] == muse ? 1.f : __builtin_amdgcn_exp2f(m[tau] - muse);
        float p[KB][4];
#pragma unroll
        for (int kblk = 0; kblk < KB; ++kblk)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                p[kblk][r] = __builtin_amdgcn_exp2f(sv[kblk][r] - muse);
        float psum = (p[0][0] + p[0][1]) + (p[0][2] + p[0][3]);
        if constexpr (KB == 2)
            psum = psum + ((p[1][0] + p[1][1]) + (p[1][2] + p[1][3]));
        psum = psum + xor16_f(psum);
        psum = psum + xor32_f(psum);
        l[tau] = l[tau] * al + psum;
        m[tau] = mnew;
        alpha[tau] = al;
        if constexpr (FP8) {
#pragma unroll
            for (int kblk = 0; kblk < KB; ++kblk)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    p[kblk][r] = p[kblk][r] * (kblk ? vs1 : vs0);
        }
#pragma unroll
        for (int kblk = 0; kblk < KB; ++kblk) {
            pa[tau][2 * kblk + 0] = pack_bf16(p[kblk][0], p[kblk][1]);
            pa[tau][2 * kblk + 1] = pack_bf16(p[kblk][2], p[kblk][3]);
        }
    }

    // Rescale O rows (slot 4*kb + r) by their slot's alpha; skipping a
    // multiply by exactly 1 changes nothing (ILP: always multiplied, so
    // the tile has no branch and the tiles of a ring round share one
    // scheduling block).
#pragma unroll
    for (int tau = 0; tau < NT; ++tau) {
        if (ILP || __builtin_amdgcn_ballot_w64(alpha[tau] != 1.f)) {
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
    // the key described at load_tile.
    // bf16: key pairs (2u, 2u + 1) of one element are gathered from the rows'
    // bf16 pairs.  fp8: the two keys' code bytes of two elements are gathered
    // first, then each half widens to that bf16 pair (exact either way).
    uint32_t vb[FP8 ? 1 : G::KEYS][G::DB / 2];  // bf16 pairs: dword w = elements 2w, 2w+1
    uint32_t vp8[FP8 ? G::DB : 1][2 * KB];      // fp8: B dword of element jb, key pair u
    if constexpr (FP8) {
#pragma unroll
        for (int u = 0; u < 2 * KB; ++u)
#pragma unroll
            for (int w = 0; w < G::VDW; ++w) {
                // bytes: key 2u, key 2u + 1 of element 4w, then of 4w + 1 (x);
                // of 4w + 2 and 4w + 3 (y)
                const uint32_t x = __builtin_amdgcn_perm(t.v[2 * u + 1][w], t.v[2 * u][w], 0x05010400u);
                const uint32_t y = __builtin_amdgcn_perm(t.v[2 * u + 1][w], t.v[2 * u][w], 0x07030602u);
                vp8[4 * w + 0][u] = fp8x2_to_bf16x2<false>(x);
                vp8[4 * w + 1][u] = fp8x2_to_bf16x2<true>(x);
                vp8[4 * w + 2][u] = fp8x2_to_bf16x2<false>(y);
                vp8[4 * w + 3][u] = fp8x2_to_bf16x2<true>(y);
            }
    } else {
#pragma unroll
        for (int i = 0; i < G::KEYS; ++i)
#pragma unroll
            for (int w = 0; w < G::VDW; ++w)
                vb[i][w] = t.v[i][w];
    }
#pragma unroll
    for (int jb = 0; jb < G::DB; ++jb) {
        const uint32_t sel = (jb & 1) ? 0x07060302u : 0x05040100u;
        uint32_t b[2 * KB];
#pragma unroll
        for (int u = 0; u < 2 * KB; ++u) {
            if constexpr (FP8)
                b[u] = vp8[jb][u];
            else
                b[u] = __builtin_amdgcn_perm(vb[2 * u + 1][jb >> 1], vb[2 * u][jb >> 1], sel);
        }
#pragma unroll
        for (int tau = 0; tau < NT; ++tau) {
            if constexpr (KB == 2) {
                const u32x4 pv = {pa[tau][0], pa[tau][1], pa[tau][2], pa[tau][3]};
                const u32x4 bv = {b[0], b[1], b[2], b[3]};
                O[tau][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, pv), __builtin_bit_cast(bf16x8, bv), O[tau][jb], 0,
                    0, 0);
            } else {
                const u32x2 pv = {pa[tau][0], pa[tau][1]};
                const u32x2 bv = {b[0], b[1]};
                O[tau][jb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                    __builtin_bit_cast(s16x4, pv), __builtin_bit_cast(s16x4, bv), O[tau][jb], 0,
                    0, 0);
            }
        }
    }
}

__device__ __forceinline__ bool ctx_ok(int C, int R, int64_t cap) { return C >= R && (int64_t)C <= cap; }

// A work item resolved to its sequence, split and kv head.
struct Item {
    int s, j, kh, C, t0, t1, npg;
    int lo;    // first key the item's rows may attend (window / floor), <= t0 + KT - 1
    int tau0;  // first slot tile of the call that the item covers
};

// First key position row `pos` attends: its sliding window (window > 0)
// and the sequence's runtime floor, whichever is later.
__device__ __forceinline__ int key_floor(int pos, int window, int floor_s)
{
    return max(floor_s, window > 0 ? pos - window + 1 : 0);
}

// Items are numbered full splits first (sequence, split, kv head), then the
// partial last splits, longest first (sequence order `s_ord`, kv head).
// s_pre: exclusive prefix over sequences of their full items; s_lo: the
// first key each sequence's first row attends (-1: no items).
template <int KT, int NT, int CH>
__device__ __forceinline__ Item resolve_item(const int* s_pre, const int* s_ord, const int* s_len,
                                             const int* s_lo, int S, int Hk, int slices,
                                             int item_in)
{
    // `slices` consecutive item numbers share one (sequence, split, kv
    // head) and take NT slot tiles each.
    const int item = item_in / slices;
    const int tau0 = (item_in - item * slices) * NT;
    const int nfull = s_pre[S];
    Item it;
    int s, local;
    if (item < nfull) {
        int lo = 0, hi = S - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_pre[mid] <= item)
                lo = mid;
            else
                hi = mid - 1;
        }
        s = __builtin_amdgcn_readfirstlane(lo);
        local = __builtin_amdgcn_readfirstlane(item - s_pre[s]);
    } else {
        const int rank = (item - nfull) / Hk;
        s = __builtin_amdgcn_readfirstlane(s_ord[rank]);
        local = item - nfull - rank * Hk;
    }
    it.s = s;
    it.C = __builtin_amdgcn_readfirstlane(s_len[s]);
    const int lo_s = max(__builtin_amdgcn_readfirstlane(s_lo[s]), 0);
    const int j0 = lo_s / CH;  // the sequence's first split with keys to attend
    const bool full = item < nfull;
    it.j = full ? j0 + local / Hk : it.C / CH;
    it.kh = full ? local - (local / Hk) * Hk : local;
    // Tiles keep their absolute grid (a multiple of KT from the split start)
    // whatever the window, so a row's arithmetic does not depend on it.
    const int base = it.j * CH;
    it.lo = max(lo_s, base);
    it.t0 = base + ((it.lo - base) / KT) * KT;
    it.t1 = min(base + CH, it.C);
    it.npg = (it.t1 - it.t0 + 15) >> 4;
    it.tau0 = __builtin_amdgcn_readfirstlane(tau0);
    return it;
}

// Lane e < npg receives block-table entry e of the item (0 elsewhere, and
// everywhere if `live` is false).
__device__ __forceinline__ int fetch_pages(const SplitArgs& a, const Item& it, bool live)
{
    const int32_t* row = a.block_table + (int64_t)it.s * a.max_pages + (it.t0 >> 4);
    const __amdgpu_buffer_rsrc_t r = rsrc(row, live ? (uint32_t)it.npg * 4u : 0u);
    const int lane = threadIdx.x & 63;
    return (int)__builtin_amdgcn_raw_buffer_load_b32(r, (uint32_t)lane * 4u, 0, 0);
}

// LDS tile ring (LR): the form of the split kernel for bf16 at head_dim 256
// with two slot tiles per item (verify rounds).  Each wave keeps its tile
// stream in two 16-KiB LDS slots filled by buffer loads that write LDS
// directly, two tiles ahead of the compute; a tile is copied into registers
// just before it is computed, and its slot is refilled at once.  A register
// ring of two-slot-tile items would not fit beside their query operands and
// accumulators (one tile in flight instead of two), and one slot tile per
// item would stream every key twice (two sibling items), which halves the
// distinct bytes in flight.  The arithmetic is the register form's.
// Batches of at most kMaxSeqLR sequences: the work list shares the LDS.
constexpr int kMaxSeqLR = 512;

#define LDS __attribute__((address_space(3)))

// The two slots of a wave's LDS ring (TB bytes each), separate LDS arrays so
// that the compiler can tell a load into one slot from a read of the other.
template <int TB, int SLOT>
__device__ __forceinline__ LDS char* lds_slot(int wave)
{
    __shared__ __attribute__((aligned(1024))) char ring[kWaves * TB];
    return (LDS char*)ring + wave * TB;
}

// A 16-byte-per-lane buffer load that writes LDS directly: lane i's bytes
// land at dst + 16 i (1 KiB per load); lanes past the resource write zeros.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, LDS char* dst, uint32_t off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS void*)dst, 16, off, 0, 0, 0);
}

// Waits on this wave's counters, with the compiler kept from moving memory
// accesses across (gfx9 s_waitcnt encoding: vmcnt bits 3:0 and 15:14,
// expcnt 6:4, lgkmcnt 11:8).  vm_wait<N>: all but the N newest vector-memory
// accesses have completed (they complete in issue order).  lds_wait: every
// LDS access has completed.
template <int N>
__device__ __forceinline__ void vm_wait()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
    __asm__ volatile("" ::: "memory");
}
__device__ __forceinline__ void lds_wait()
{
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
    __asm__ volatile("" ::: "memory");
}

// ILP (calls with at most one work item per wave, where a tile's time is
// the wave's own instruction stream): the tile loop has no branch -- the
// rescale is always applied, a main-loop tile is never a padding tile and
// the tiles of an item with a page outside the pool (such pages load
// nothing) are computed and their result replaced by NaN as in the other
// form -- so the compiler interleaves the tiles of a ring round.  Same bits.
template <int D, bool FP8, int NT, bool WIN, bool SSC, bool LR, bool ILP>
__global__ __launch_bounds__(256, (Plan<D, FP8, NT>::OCC)) void split_kernel(SplitArgs a)
{
    static_assert(!SSC || FP8, "scalar-unit scales: fp8 only");
    static_assert(!LR || (D == 256 && !FP8 && NT == 2),
                  "LDS ring: bf16, head_dim 256, two slot tiles");
    using G = Geo<D, FP8>;
    // Ring period (items are padded to a multiple of it) and depth.
    constexpr int NBUF = LR ? 2 : Plan<D, FP8, NT>::NBUF;
    constexpr bool PREQ = Plan<D, FP8, NT>::PREQ;
    constexpr int KT = G::KT;
    static_assert(G::CHUNK / 16 <= 64, "one lane per partial-split length class");
    constexpr int MS = LR ? kMaxSeqLR : kMaxSeq;
    __shared__ int s_pre[MS + 1];  // full items before each sequence
    __shared__ int s_ord[MS];      // sequences with a partial split, longest first
    __shared__ int s_len[MS];
    __shared__ int s_lo[MS];  // first key the sequence's first row attends, -1: none
    // [0, 64): sequences per length class; [64, 128): placed so far; [128,
    // 192): sequences of longer classes; [192, 196): per-wave item sums.
    // Class c (1 .. CHUNK/16) is entry c - 1.
    __shared__ __attribute__((aligned(16))) int s_cls[256];
    __shared__ int s_cnt[2][256];  // per group of 256 sequences: class counts per wave
    __shared__ int s_npart;        // partial items

    const int S = a.n_seq, R = a.rows, Hk = a.n_head_kv, H = a.n_head;
    const int g = H / Hk, ppt = 16 / g;
    const int64_t cap = (int64_t)a.max_pages * 16;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // The work list, built in LDS by every workgroup alike (item set-up then
    // waits on no global load): lengths, first keys, the exclusive prefix
    // over sequences of their full items, and the order of the partial last
    // splits -- by length class (pages) from the longest, and by sequence
    // within a class (a stable counting sort).  With full items first and
    // each wave taking the items of rounds in alternating directions, the
    // longest partial items go to the waves with the least work, and the
    // last items of the grid are the shortest.
    {
        // lo: first key of the sequence's first row; -1 marks a sequence
        // whose floor lies outside 0 .. that row's position (no items, NaN).
        auto first_key = [&](int s, int C) {
            const int f = a.kv_floor ? a.kv_floor[s] : 0;
            if (f < 0 || f > C - R)
                return -1;
            return key_floor(C - R, a.window, f);
        };
        auto nfull = [&](int C, int lo) {
            if (lo < 0)
                return 0;
            const int end = a.below_round ? (C - R) / G::CHUNK : C / G::CHUNK;
            return max(end - lo / G::CHUNK, 0) * Hk;
        };
        // Length class of a sequence's partial split (0: it has none).
        auto pclass = [&](int C, int lo) {
            if (a.below_round || lo < 0 || C % G::CHUNK == 0)
                return 0;
            return (C - max(lo, C - C % G::CHUNK) + 15) >> 4;
        };
        if (tid < 128)
            s_cls[tid] = 0;
        const int per = (S + 255) / 256;
        const int b0 = tid * per;
        int loc = 0;
        for (int i = 0; i < per; ++i) {
            const int s = b0 + i;
            if (s < S) {
                const int C = a.ctx_lens[s];
                const int lo = ctx_ok(C, R, cap) ? first_key(s, C) : -1;
                s_len[s] = C;
                s_lo[s] = lo;
                loc += nfull(C, lo);
            }
        }
        int inc = loc;  // inclusive prefix over the wave's threads
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(inc, d, 64);
            inc += lane >= d ? v : 0;
        }
        if (lane == 63)
            s_cls[192 + wave] = inc;
        __syncthreads();
        int run = inc - loc;
        for (int w = 0; w < wave; ++w)
            run += s_cls[192 + w];
        for (int i = 0; i < per; ++i) {
            const int s = b0 + i;
            if (s < S) {
                const int C = s_len[s], lo = s_lo[s];
                s_pre[s] = run;
                run += nfull(C, lo);
                const int c = pclass(C, lo);
                if (c > 0)
                    atomicAdd(&s_cls[c - 1], 1);
            }
        }
        if (tid == 255)
            s_pre[S] = run;  // the last thread's range ends the list
        __syncthreads();
        if (tid < 64) {
            int longer = 0;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const i32x4 v = *(const i32x4*)&s_cls[4 * q];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    longer += 4 * q + e > tid ? v[e] : 0;
            }
            s_cls[128 + tid] = longer;
            if (tid == 0)
                s_npart = (longer + s_cls[0]) * Hk;
        }
        __syncthreads();
        for (int s0 = 0, par = 0; s0 < S; s0 += 256, par ^= 1) {
            const int s = s0 + tid;
            const int c = s < S ? pclass(s_len[s], s_lo[s]) : 0;
            // Lanes of the wave in class c (same) and in class lane + 1 (mine),
            // from one ballot per bit of the class.
            uint64_t same = ~0ull, mine = ~0ull;
#pragma unroll
            for (int k = 0; k < 7; ++k) {
                const uint64_t bk = __builtin_amdgcn_ballot_w64(((c >> k) & 1) != 0);
                same &= ((c >> k) & 1) ? bk : ~bk;
                mine &= (((lane + 1) >> k) & 1) ? bk : ~bk;
            }
            const int below = (int)__builtin_amdgcn_mbcnt_hi(
                (uint32_t)(same >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)same, 0u));
            s_cnt[par][64 * wave + lane] = __builtin_popcountll(mine);
            __syncthreads();
            if (c > 0) {
                int r = s_cls[128 + c - 1] + s_cls[64 + c - 1] + below;
                for (int w = 0; w < wave; ++w)
                    r += s_cnt[par][64 * w + c - 1];
                s_ord[r] = s;
            }
            if (s0 + 256 < S) {
                __syncthreads();
                if (tid < 64)
                    s_cls[64 + tid] += s_cnt[par][tid] + s_cnt[par][64 + tid] +
                                       s_cnt[par][128 + tid] + s_cnt[par][192 + tid];
            }
        }
        __syncthreads();
    }

    const int n = lane & 15, kb = lane >> 4;
    // Wave-uniform values are made visibly uniform (scalar registers), so
    // that loop bounds, page ids and buffer resources stay scalar.
    const int total = __builtin_amdgcn_readfirstlane((s_pre[S] + s_npart) * a.slices);
    const int nwaves = gridDim.x * kWaves;
    const float sm_log2 = kLog2e / __builtin_sqrtf((float)D);
    const uint8_t* __restrict__ kp = (const uint8_t*)a.k_pool;
    const uint8_t* __restrict__ vp = (const uint8_t*)a.v_pool;
    const uint32_t koff = (uint32_t)(n * G::ROWB + 16 * kb);
    const uint32_t voff = (uint32_t)(4 * kb * G::ROWB + n * G::VPB);
    const __amdgpu_buffer_rsrc_t r_ks =
        rsrc(a.k_scale, FP8 ? (uint32_t)(a.n_pages * Hk * 4) : 0u);
    const __amdgpu_buffer_rsrc_t r_vs =
        rsrc(a.v_scale, FP8 ? (uint32_t)(a.n_pages * Hk * 4) : 0u);

    // Page e of item I: its (page, kv head) chunk and its rows inside the
    // item.  An entry outside the pool, a page past the item and a dead item
    // give chunk 0 with no rows, so no load can leave the pool.
    auto page = [&](const Item& I, int pidv, bool live, int e, int64_t& chunk, int& rows) {
        const int p = rdlane(pidv, e);
        // Pages wholly below the item's first key are neither read nor
        // checked (a runtime floor may have released them).
        const bool below = I.t0 + 16 * e + 16 <= I.lo;
        const bool ok = live && e < I.npg && !below && p >= 0 && (int64_t)p < a.n_pages;
        chunk = (int64_t)(ok ? p : 0) * Hk + I.kh;
        // (readfirstlane keeps the clamp, which only the vector unit has,
        // from turning the buffer resources into per-lane values.)
        if constexpr (ILP) {
            const int rr = __builtin_amdgcn_readfirstlane(min(16, max(0, I.t1 - (I.t0 + 16 * e))));
            rows = ok ? rr : 0;
        } else {
            rows = ok ? __builtin_amdgcn_readfirstlane(min(16, max(0, I.t1 - (I.t0 + 16 * e)))) : 0;
        }
    };
    auto issue = [&](Raw<D, FP8>& buf, const Item& I, int pidv, bool live, int tile) {
        const int e0 = tile * G::KB;
        const int e1 = G::KB == 2 ? e0 + 1 : e0;
        int64_t c0, c1;
        int r0, r1;
        page(I, pidv, live, e0, c0, r0);
        page(I, pidv, live, e1, c1, r1);
        load_tile<D, FP8>(buf, kp, vp, c0, c1, r0, r1, koff, voff);
    };
    // Query operands of item I; empty slots read past the end of the query
    // rows of I's sequence and get zeros.
    auto load_q = [&](u32x4 (&qd)[NT][G::STEPS], const Item& I, bool live) {
        const uint16_t* qs = (const uint16_t*)a.q + (int64_t)I.s * R * H * D;
        const __amdgpu_buffer_rsrc_t rq = rsrc(qs, live ? (uint32_t)(R * H * D * 2) : 0u);
        const int cm = (I.C - R) % ppt;
        const int h = I.kh * g + (n % g);
#pragma unroll
        for (int tau = 0; tau < NT; ++tau) {
            const int r = slot_row(n, I.tau0 + tau, g, ppt, R, cm);
            const uint32_t qo = r >= 0 ? (uint32_t)((r * H + h) * D) * 2u : kFar;
#pragma unroll
            for (int st = 0; st < G::STEPS; ++st)
                qd[tau][st] = __builtin_amdgcn_raw_buffer_load_b128(
                    rq, qo + 2u * (uint32_t)qk_dmap<D, FP8>(st, kb), 0, 0);
        }
    };
    // fp8 page scales, two ways.  SSC: each tile's K and V page scales by
    // the scalar unit, issued after the compute that precedes them in the
    // ring (the scalar counter completes out of order, so a compute's wait
    // for its own scales waits for every scalar load issued before it) and
    // used NBUF - 1 tiles later; kept raw with their pages' rows in the
    // item, the zero for an empty page chosen at the compute.  This frees
    // the vector memory path of the per-item loads below (two 64-lane loads
    // touching 64 scattered lines each), but puts a scalar round trip within
    // one tile of each compute: for calls with many items per wave.
    const __attribute__((address_space(4))) float* ksp =
        (const __attribute__((address_space(4))) float*)a.k_scale;
    const __attribute__((address_space(4))) float* vsp =
        (const __attribute__((address_space(4))) float*)a.v_scale;
    float sk[NBUF][2], sv[NBUF][2];  // (SSC) raw scales of each ring tile's pages
    int sr[NBUF][2];                 // (SSC) rows of those pages in their item
    auto issue_sc = [&](int slot, const Item& I, int pidv, bool live, int tile) {
        if constexpr (SSC) {
            const int e0 = tile * G::KB;
            const int e1 = G::KB == 2 ? e0 + 1 : e0;
            int64_t c0, c1;
            page(I, pidv, live, e0, c0, sr[slot][0]);
            page(I, pidv, live, e1, c1, sr[slot][1]);
            __builtin_amdgcn_sched_barrier(0);
            sk[slot][0] = ksp[c0];
            sv[slot][0] = vsp[c0];
            sk[slot][1] = ksp[c1];
            sv[slot][1] = vsp[c1];
        }
    };
    // Otherwise per item: lane e holds page e's scales (zero past the item,
    // for a page wholly below the item's first key -- a runtime floor may
    // have released its entry, which may then name any page -- for an entry
    // outside the pool, and for bf16).  A zero V scale keeps the masked
    // keys' zero probabilities zero.
    auto load_scales = [&](float& ks, float& vs, const Item& I, int pidv, bool live) {
        ks = vs = 0.f;
        if constexpr (FP8 && !SSC) {
            const bool ok = live && lane < I.npg && I.t0 + 16 * lane + 16 > I.lo && pidv >= 0 &&
                            (int64_t)pidv < a.n_pages;
            const uint32_t so = ok ? (uint32_t)(pidv * Hk + I.kh) * 4u : kFar;
            ks = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_ks, so, 0, 0));
            vs = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_vs, so, 0, 0));
        }
    };

    // Wave w takes item w of round 0, then of each round r the item at
    // w from the round's start (r even) or from its end (r odd).  Item
    // numbers grow with the round, so a wave's items end at its first round
    // past the list.
    const int wid = __builtin_amdgcn_readfirstlane(blockIdx.x * kWaves + wave);
    auto item_of = [&](int r) { return r * nwaves + ((r & 1) ? nwaves - 1 - wid : wid); };
    int round = 0;
    int item = item_of(0);
    if (item >= total)
        return;

    // The wave's tiles form one stream over its items: the ring's loads run
    // NBUF - 1 tiles ahead of the compute, across item boundaries.  Items
    // are padded to a multiple of NBUF tiles (padding tiles load nothing and
    // are not computed), so every item starts at ring slot 0.
    // Table entries are fetched two items ahead and held in registers one
    // item ahead, so the ring never waits for them.
    Item cur = resolve_item<KT, NT, G::CHUNK>(s_pre, s_ord, s_len, s_lo, S, Hk, a.slices, item);
    int pid = fetch_pages(a, cur, true);
    bool has_next = item_of(1) < total;
    Item nxt = resolve_item<KT, NT, G::CHUNK>(s_pre, s_ord, s_len, s_lo, S, Hk, a.slices,
                                             has_next ? item_of(1) : item);
    int pid_n = fetch_pages(a, nxt, has_next);
    // A full wait (never too weak): the loop then finds pid and pid_n
    // resolved on entry as it does on every later iteration, and its
    // compiler-placed waits need not cover these loads.
    __builtin_amdgcn_s_waitcnt(0);
    u32x4 qop[NT][G::STEPS];
    float ksc, vsc;
    load_q(qop, cur, true);
    load_scales(ksc, vsc, cur, pid, true);
    // (LR) A tile's 16 loads, each 1 KiB of the slot (lane i's 16 bytes at
    // 16 i): the K pieces, then the V row pieces, in load_tile's order; read
    // back by the same lanes into the same registers.
    using LDSP = LDS char*;
    constexpr int NLD = G::KLD + 4 * (G::VDW / 4);
    constexpr int TB = NLD * 1024;
    LDSP r0 = nullptr;
    LDSP r1 = nullptr;
    if constexpr (LR) {
        r0 = lds_slot<TB, 0>(__builtin_amdgcn_readfirstlane(wave));
        r1 = lds_slot<TB, 1>(__builtin_amdgcn_readfirstlane(wave));
    }
    auto issue_l = [&](LDSP slot, const Item& I, int pidv, bool live, int tile) {
        if constexpr (LR) {
            int64_t c0;
            int n0;
            page(I, pidv, live, tile, c0, n0);
            const uint32_t nb = (uint32_t)(n0 * G::ROWB);
            const __amdgpu_buffer_rsrc_t rk = rsrc(kp + c0 * G::CHUNKB, nb);
            const __amdgpu_buffer_rsrc_t rv = rsrc(vp + c0 * G::CHUNKB, nb);
#pragma unroll
            for (int c = 0; c < G::KLD; ++c)
                load_lds16(rk, slot + 1024 * c, koff + 64 * c);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int c = 0; c < G::VDW / 4; ++c)
                    load_lds16(rv, slot + 1024 * (G::KLD + (G::VDW / 4) * i + c),
                               voff + i * G::ROWB + 16 * c);
        }
    };
    auto read_l = [&](Raw<D, FP8>& t, LDSP slot) {
        if constexpr (LR) {
            typedef LDS u32x4* LQ;
#pragma unroll
            for (int c = 0; c < G::KLD; ++c)
                t.k[0][c] = *(LQ)(slot + 1024 * c + 16 * lane);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int c = 0; c < G::VDW / 4; ++c) {
                    const int j = G::KLD + (G::VDW / 4) * i + c;
                    const u32x4 w = *(LQ)(slot + 1024 * j + 16 * lane);
                    t.v[i][4 * c + 0] = w[0];
                    t.v[i][4 * c + 1] = w[1];
                    t.v[i][4 * c + 2] = w[2];
                    t.v[i][4 * c + 3] = w[3];
                }
        }
    };

    Raw<D, FP8> buf[LR ? 1 : NBUF];
    if constexpr (LR) {
        issue_l(r0, cur, pid, true, 0);
        issue_l(r1, cur, pid, true, 1);
    } else {
#pragma unroll
        for (int k = 0; k < NBUF - 1; ++k) {
            issue(buf[k], cur, pid, true, k);
            issue_sc(k, cur, pid, true, k);
        }
    }

    for (;;) {
        // The item after next: geometry and table entries now.
        const int next2 = item_of(round + 2);
        const bool has_next2 = next2 < total;
        const Item nxt2 = resolve_item<KT, NT, G::CHUNK>(s_pre, s_ord, s_len, s_lo, S, Hk,
                                                        a.slices, has_next2 ? next2 : item);
        const int pid_nn = fetch_pages(a, nxt2, has_next2);

        const int s = cur.s, j = cur.j, kh = cur.kh, C = cur.C, t0 = cur.t0, t1 = cur.t1;
        const int npg = cur.npg;
        const int cmr_mod = (C - R) % ppt;
        const int f_s = a.kv_floor ? __builtin_amdgcn_readfirstlane(a.kv_floor[s]) : 0;
        const bool badp = lane < npg && t0 + 16 * lane + 16 > cur.lo &&
                          (pid < 0 || (int64_t)pid >= a.n_pages);
        const bool bad = __builtin_amdgcn_ballot_w64(badp) != 0;
        const int nt = (t1 - t0 + KT - 1) / KT;
        const int ntp = (nt + NBUF - 1) / NBUF * NBUF;

        int first[NT], last[NT];
        float m[NT], l[NT];
        f32x4 O[NT][G::DB];
#pragma unroll
        for (int tau = 0; tau < NT; ++tau) {
            const int r = slot_row(n, cur.tau0 + tau, g, ppt, R, cmr_mod);
            last[tau] = r >= 0 ? C - R + r : -1;
            first[tau] = r >= 0 ? key_floor(C - R + r, a.window, f_s) : 0;
            m[tau] = neg_inf();
            l[tau] = 0.f;
#pragma unroll
            for (int jb = 0; jb < G::DB; ++jb)
                O[tau][jb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        auto kscale = [&](int e) {
            return FP8 ? rdlane_f(ksc, e < npg ? e : 0) * sm_log2 : sm_log2;
        };
        auto vscale = [&](int e) { return FP8 ? rdlane_f(vsc, e < npg ? e : 0) : 1.f; };
        auto compute = [&](const Raw<D, FP8>& t, int tile, int slot) {
            const int e0 = tile * G::KB;
            const int e1 = G::KB == 2 ? e0 + 1 : e0;
            if constexpr (SSC) {
                constexpr int L = G::KB - 1;
                compute_tile<D, FP8, NT, WIN, ILP>(
                    t, qop, first, last, m, l, O, t0 + KT * tile,
                    (sr[slot][0] > 0 ? sk[slot][0] : 0.f) * sm_log2,
                    (sr[slot][L] > 0 ? sk[slot][L] : 0.f) * sm_log2,
                    sr[slot][0] > 0 ? sv[slot][0] : 0.f, sr[slot][L] > 0 ? sv[slot][L] : 0.f, kb);
            } else {
                compute_tile<D, FP8, NT, WIN, ILP>(t, qop, first, last, m, l, O, t0 + KT * tile,
                                              kscale(e0), kscale(e1), vscale(e0), vscale(e1),
                                              kb);
            }
        };

        // Tiles whose ring successor is still in this item.
        for (int it = 0; it < ntp - NBUF; it += NBUF) {
#pragma unroll
            for (int k = 0; k < NBUF; ++k) {
                const int tile = it + k;
                if constexpr (LR) {
                    // Tile `tile` is in slot k, tile + 1 in the other slot.
                    vm_wait<NLD>();
                    read_l(buf[0], k ? r1 : r0);
                    lds_wait();
                    issue_l(k ? r1 : r0, cur, pid, true, tile + 2);
                    if (!bad && tile < nt)
                        compute(buf[0], tile, k);
                } else {
                    issue(buf[(k + NBUF - 1) % NBUF], cur, pid, true, tile + NBUF - 1);
                    if (ILP || (!bad && tile < nt))
                        compute(buf[k], tile, k);
                    issue_sc((k + NBUF - 1) % NBUF, cur, pid, true, tile + NBUF - 1);
                }
            }
        }
        // The item's last NBUF tiles; the ring moves on to the next item,
        // whose scales (and query rows) are loaded first.
        u32x4 qop_n[PREQ ? NT : 1][G::STEPS];
        float ksc_n, vsc_n;
        if constexpr (PREQ)
            load_q(qop_n, nxt, has_next);
        load_scales(ksc_n, vsc_n, nxt, pid_n, has_next);
#pragma unroll
        for (int k = 0; k < NBUF; ++k) {
            const int tile = ntp - NBUF + k;
            if constexpr (LR) {
                vm_wait<NLD>();
                read_l(buf[0], k ? r1 : r0);
                lds_wait();
                issue_l(k ? r1 : r0, nxt, pid_n, has_next, k);
                if (!bad && tile < nt)
                    compute(buf[0], tile, k);
            } else {
                if (k == 0)
                    issue(buf[NBUF - 1], cur, pid, true, ntp - 1);
                else
                    issue(buf[k - 1], nxt, pid_n, has_next, k - 1);
                if (!bad && tile < nt)
                    compute(buf[k], tile, k);
                if (k == 0)
                    issue_sc(NBUF - 1, cur, pid, true, ntp - 1);
                else
                    issue_sc(k - 1, nxt, pid_n, has_next, k - 1);
            }
        }

        // Partials: O rows are slots 4*kb + r; m, l of slot n.  Bounds-checked
        // stores: an empty slot stores at kFar, which the resource drops, so
        // no store sits under a branch either.
        const float qnan = __builtin_nanf("");
        const int64_t rs = (int64_t)a.max_split * H;  // records per row
        const int64_t rec0 = (int64_t)s * R * rs + (int64_t)j * H;  // record (s, row 0, j, head 0)
        const int64_t nrec = (R - 1) * rs + H;  // through record (s, R - 1, j, H - 1)
        const __amdgpu_buffer_rsrc_t ro = rsrc(a.o_part + rec0 * D, (uint32_t)(nrec * D * 4));
        const __amdgpu_buffer_rsrc_t rml = rsrc(a.ml_part + rec0 * 2, (uint32_t)(nrec * 2 * 4));
#pragma unroll
        for (int tau = 0; tau < NT; ++tau) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int slot = 4 * kb + r;
                const int row = slot_row(slot, cur.tau0 + tau, g, ppt, R, cmr_mod);
                const int h = kh * g + (slot % g);
                const uint32_t off =
                    row >= 0 ? (uint32_t)(((row * rs + h) * D + n * G::DB) * 4) : kFar;
#pragma unroll
                for (int jb = 0; jb < G::DB; jb += 4) {
                    const f32x4 v = bad ? f32x4{qnan, qnan, qnan, qnan}
                                        : f32x4{O[tau][jb][r], O[tau][jb + 1][r],
                                                O[tau][jb + 2][r], O[tau][jb + 3][r]};
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ro,
                                                           off + 4u * jb, 0, 0);
                }
            }
            const int row = slot_row(n, cur.tau0 + tau, g, ppt, R, cmr_mod);
            const int h = kh * g + (n % g);
            const uint32_t off = (kb == 0 && row >= 0) ? (uint32_t)((row * rs + h) * 8) : kFar;
            const f32x2 v = bad ? f32x2{qnan, qnan} : f32x2{m[tau], l[tau]};
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), rml, off, 0, 0);
        }

        if (!has_next)
            break;
        ++round;
        item = item_of(round);
        cur = nxt;
        pid = pid_n;
        nxt = nxt2;
        pid_n = pid_nn;
        has_next = has_next2;
        if constexpr (PREQ) {
#pragma unroll
            for (int tau = 0; tau < NT; ++tau)
#pragma unroll
                for (int st = 0; st < G::STEPS; ++st)
                    qop[tau][st] = qop_n[tau][st];
        } else {
            load_q(qop, cur, true);
        }
        ksc = ksc_n;
        vsc = vsc_n;
    }
    // (LR) The last tiles' loads (of no item: they write zeros) land before
    // the wave ends and its LDS can be given to another workgroup.
    if constexpr (LR)
        __builtin_amdgcn_s_waitcnt(0);
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
    const int f_s = a.kv_floor ? a.kv_floor[s] : 0;
    if (f_s < 0 || f_s > C - R) {
#pragma unroll
        for (int e = 0; e < E; ++e)
            out[e] = 0x7FC0;  // NaN
        return;
    }
    const int pos = C - R + r;
    const int ns = (pos >> a.chunk_log2) + 1;
    const int jlo = key_floor(pos, a.window, f_s) >> a.chunk_log2;  // first split the row attends
    const int64_t rec = ((int64_t)s * R + r) * a.max_split * H + h;  // record (s, r, 0, h)
    const float* ml = a.ml_part + rec * 2;
    const float* op = a.o_part + rec * D + lane * E;
    const int64_t mls = (int64_t)H * 2, ops = (int64_t)H * D;  // per-split strides

    // Splits in groups of 64, lane = split within the group.
    float M = neg_inf();
    bool nan = false;
    const int jstart = jlo & ~63;
    for (int j0 = jstart; j0 < ns; j0 += 64) {
        const int jj = j0 + lane;
        const float mj = jj < ns && jj >= jlo ? ml[jj * mls] : neg_inf();
        nan |= mj != mj;
        M = fmaxf(M, mj);
    }
    nan = __builtin_amdgcn_ballot_w64(nan) != 0;
#pragma unroll
    for (int k = 1; k < 64; k <<= 1)
        M = fmaxf(M, shfl_xor_f(M, k));

    float num[E], den = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e)
        num[e] = 0.f;
    for (int j0 = jstart; j0 < ns; j0 += 64) {
        const int jj = j0 + lane;
        float wj = 0.f, lj = 0.f;
        if (jj < ns && jj >= jlo) {
            const f32x2 v = *(const f32x2*)(ml + jj * mls);
            wj = v[0] == M ? 1.f : __builtin_amdgcn_exp2f(v[0] - M);
            lj = v[1];
        }
        float dl = wj * lj;
#pragma unroll
        for (int k = 1; k < 64; k <<= 1)
            dl = dl + shfl_xor_f(dl, k);
        den = den + dl;
        const int cnt = min(64, ns - j0);
        const float* o0 = op + (int64_t)j0 * ops;
        int q = max(0, jlo - j0);
        for (; q + 8 <= cnt; q += 8) {
            float ov[8][E];
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int e = 0; e < E; ++e)
                    ov[u][e] = o0[(int64_t)(q + u) * ops + e];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const float wu = rdlane_f(wj, q + u);
#pragma unroll
                for (int e = 0; e < E; ++e)
                    num[e] = num[e] + wu * ov[u][e];
            }
        }
        for (; q < cnt; ++q) {
            const float wu = rdlane_f(wj, q);
#pragma unroll
            for (int e = 0; e < E; ++e)
                num[e] = num[e] + wu * o0[(int64_t)q * ops + e];
        }
    }
#pragma unroll
    for (int e = 0; e < E; ++e)
        out[e] = nan ? (uint16_t)0x7FC0 : (uint16_t)bf16_bits(num[e] / den);
}

template <int D, bool FP8, int NT, bool WIN, bool LR = false>
hipError_t launch_split_t(const SplitArgs& a0, hipStream_t stream)
{
    using G = Geo<D, FP8>;
    static_assert((G::CHUNK & (G::CHUNK - 1)) == 0, "split size: a power of two");
    SplitArgs a = a0;
    a.chunk_log2 = __builtin_ctz((unsigned)G::CHUNK);
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
        if constexpr (LR)
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &per, split_kernel<D, FP8, NT, WIN, false, true, false>, 256, 0);
        else
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &per, split_kernel<D, FP8, NT, WIN, false, false, false>, 256, 0);
        if (e != hipSuccess)
            return e;
        // 1024-key splits: one workgroup per CU keeps about as many items per
        // wave as 512-key splits at two (the load stream is as fast).
        if (G::CHUNK > kChunk && per > 1)
            per = 1;
        grid_cap = cus * (per > 0 ? per : 1);
    }
    const int Hk = a.n_head_kv;
    const int64_t upper = (int64_t)a.n_seq * a.max_split * Hk * a.slices;  // items, at most
    int64_t blocks = (upper + kWaves - 1) / kWaves;
    if (blocks > grid_cap)
        blocks = grid_cap;
    if (a.max_blocks > 0 && blocks > a.max_blocks)
        blocks = a.max_blocks;
    if (blocks < 1)
        blocks = 1;
    // Scalar-unit page scales (fp8, four-deep ring) where the waves have many
    // items each: at least two (sequence, kv head) streams per wave.  Both
    // forms compute the same bits.
    constexpr bool CAN_SSC = FP8 && Plan<D, FP8, NT>::NBUF == 4;
    const bool ssc = CAN_SSC && (int64_t)a.n_seq * Hk * a.slices >= 2 * blocks * kWaves;
    // The branch-free tile loop where every wave has at most one item
    // (decode without a window).  Both forms compute the same bits.
    constexpr bool CAN_ILP = NT == 1 && !WIN && !LR;
    const bool ilp = CAN_ILP && upper <= blocks * kWaves;
    if (a.phase != 2) {
        if (a.ev_start)
            (void)hipEventRecord(a.ev_start, stream);
        if constexpr (LR) {
            hipLaunchKernelGGL((split_kernel<D, FP8, NT, WIN, false, true, false>),
                               dim3((unsigned)blocks), dim3(256), 0, stream, a);
        } else if (CAN_ILP && ilp) {
            if constexpr (CAN_ILP)
                hipLaunchKernelGGL((split_kernel<D, FP8, NT, WIN, false, false, true>),
                                   dim3((unsigned)blocks), dim3(256), 0, stream, a);
        } else if constexpr (CAN_SSC) {
            if (ssc)
                hipLaunchKernelGGL((split_kernel<D, FP8, NT, WIN, true, false, false>),
                                   dim3((unsigned)blocks), dim3(256), 0, stream, a);
            else
                hipLaunchKernelGGL((split_kernel<D, FP8, NT, WIN, false, false, false>),
                                   dim3((unsigned)blocks), dim3(256), 0, stream, a);
        } else {
            hipLaunchKernelGGL((split_kernel<D, FP8, NT, WIN, false, false, false>),
                               dim3((unsigned)blocks), dim3(256), 0, stream, a);
        }
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        if (a.ev_stop)
            (void)hipEventRecord(a.ev_stop, stream);
    }
    if (a.phase == 1)
        return hipSuccess;
    const int64_t waves = (int64_t)a.n_seq * a.rows * a.n_head;
    hipLaunchKernelGGL((combine_kernel<D>), dim3((unsigned)((waves + kWaves - 1) / kWaves)),
                       dim3(256), 0, stream, a);
    return hipGetLastError();
}

// Slot tiles per work item for a call needing `nt` tiles: the rest of the
// call's tiles go to sibling items (consecutive numbers, the same keys, so
// the second read of a tile comes from L2).  A row's arithmetic is the same
// in any tile of any instantiation, so this changes no bit of the output.
// Measured: at head_dim 128 two tiles per item beat one (fp8, 8 rows x 4
// heads) and four (bf16, 8 rows x 8 heads: 514 -> 299 us); at head_dim 256
// with the register ring one tile per item equals two (two tiles leave
// room for one tile in flight).  bf16 at head_dim 256 with two or more
// tiles takes the LDS-ring form with two tiles per item where the batch
// fits its work list.
template <int D>
int kernel_tiles(int nt)
{
    return D == 256 ? 1 : (nt < 2 ? nt : 2);
}

template <int D, bool FP8, bool WIN>
hipError_t launch_nt_w(const SplitArgs& a0, int nt, hipStream_t stream)
{
    SplitArgs a = a0;
    if constexpr (D == 256 && !FP8) {
        if (nt >= 2 && a.n_seq <= kMaxSeqLR) {
            a.slices = nt / 2;
            return launch_split_t<D, FP8, 2, WIN, true>(a, stream);
        }
    }
    const int ntk = kernel_tiles<D>(nt);
    a.slices = nt / ntk;
    switch (ntk) {
    case 1: return launch_split_t<D, FP8, 1, WIN>(a, stream);
    case 2:
        if constexpr (D <= 128)
            return launch_split_t<D, FP8, 2, WIN>(a, stream);
        return hipErrorNotSupported;
    default: return hipErrorNotSupported;
    }
}

// Calls with a window or a floor run instantiations that also compare each
// key with the row's first key; the others keep the single compare.
template <int D, bool FP8>
hipError_t launch_nt(const SplitArgs& a, int nt, hipStream_t stream)
{
    if (a.window > 0 || a.kv_floor)
        return launch_nt_w<D, FP8, true>(a, nt, stream);
    return launch_nt_w<D, FP8, false>(a, nt, stream);
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
