// prefill_pipe.hip -- the prefill chunk on a bf16 cache, or on an fp8 cache
// with both fp8 bits (QK^T and PV on the fp8 matrix unit), with the work of
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
//     output wave 4 + w         O^T += V^T . P^T for 64 rows (groups 2 (w / 2)
//                               and 2 (w / 2) + 1) and one half of head_dim
//                               (w % 2): V^T read from LDS with the
//                               transposing reads, P^T read back from LDS,
//                               rows rescaled when their score wave raised a
//                               running maximum
//   A score wave feeds every K operand it reads from LDS to two matrix
//   instructions (one per 16-row tile) and an output wave every V operand to
//   four, so the LDS bytes per flop are a half (K) and a quarter (V) of a
//   one-tile-per-wave kernel's; and each SIMD hosts one wave of each role, so
//   one wave's softmax or LDS latency overlaps the other's matrix work.
//   Roles run one tile apart: in iteration i the score waves turn tile i's
//   scores into probabilities while the output waves accumulate tile i - 1;
//   one barrier per iteration hands P, the rescale factors and the freshly
//   loaded tiles over.  Each role is also pipelined by itself: a score wave
//   computes the scores of tile i + 2 on the matrix unit while tile i's
//   softmax runs (so the softmax never waits for products queued in the
//   matrix unit behind the output wave's), and an output wave reads tile i's
//   V operands while it multiplies tile i - 1's.
//
// Tiles and buffers
//   Keys stream in 32-key tiles (two 16-token pages) through four LDS slots
//   per tensor.  In iteration i the score waves read K(i + 2) and load
//   K(i + 5) into the slot K(i + 1) left free; the output waves read V(i)
//   and load V(i + 3) into the slot V(i - 1) left free; so every tile load
//   has two iterations to land and the per-tile barrier waits only for
//   loads issued before the previous iteration.  P and the rescale factors
//   of tiles i - 1 and i sit in two more buffers.  Each wave loads 8 key
//   rows of one page per tile, by buffer loads that write LDS directly,
//   interleaved with its matrix instructions so the workgroup's waves do not
//   queue at the texture addresser together; block-table entries are read
//   with scalar loads.  The buffer descriptor of each page covers only its
//   rows below ctx_len, so rows past the context arrive as zeros; a
//   block-table entry outside the pool is never dereferenced and turns the
//   workgroup's rows to NaN.  Pages wholly below the first key any row
//   attends are not read.  K and V rows are stored row-major (bf16), each
//   row's 16-byte chunks XOR-swizzled by the row index, so the operand
//   reads of a column of rows are conflict-free.
//
// fp8 cache (both fp8 bits of the prefill_fp8 switch; "Radiance Architecture
// Plugins -- declaring a model", section "Declare: the metadata")
//   K and V tiles stay E4M3 codes in LDS (half the bytes of bf16 rows), with
//   their pages' scales beside them (scalar loads by the wave that loads the
//   page's first rows).  Score waves hold each query vector rounded to E4M3
//   at a power-of-two scale and compute S^T on
//   v_mfma_scale_f32_16x16x128_f8f6f4; the K page scale, the query's scale
//   and the softmax scale join each score in the exponent.  They write P^T as
//   E4M3 codes of p times the tile's V page scales over 2^F (F the exponent
//   of the tile's largest V scale); output waves read V^T with the
//   transposing byte reads and accumulate on v_mfma_f32_16x16x32_fp8_fp8.  O
//   is held divided by 2^F; a change of F reaches the output waves as part of
//   their rows' rescale factors, and the final 2^F joins 1 / l.
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
#include "qround.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));

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

// fp8 rows (D bytes, CK chunks of 16): the physical chunk of logical chunk
// c in the K row of key k is c ^ swzk(k), which puts the 16 rows the QK^T
// operand reads take one chunk pair from on distinct bank groups (for
// 128-byte rows, two to a bank line, on distinct halves); in the V row of
// key k (0..31) it is c ^ swzv(k), which keeps the eight rows one transposing
// byte read gathers (keys 4 kb .. + 3 and 16 + the same) on distinct chunks.
template <int CK>
__device__ __forceinline__ int swzk(int k)
{
    return CK == 16 ? (k & 15) : ((k >> 1) & 7);
}
template <int CK>
__device__ __forceinline__ int swzv(int k)
{
    return (k ^ (k >> 4)) & (CK - 1);
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

// F8: an fp8 cache whose K and V codes stay codes in LDS (QK^T and PV on
// the fp8 matrix unit).
template <int D, bool F8>
struct PGeo {
    static constexpr int ROWL = (F8 ? 1 : 2) * D;   // bytes of one key row (pool and LDS)
    static constexpr int TILEB = kKT * ROWL;        // one K (or V) tile in LDS
    static constexpr int KSTEPS = D / 32;           // k-steps of QK^T (bf16)
    static constexpr int QS = D / 128;              // k-steps of QK^T (fp8)
    static constexpr int DBLK = D / 16;             // 16-wide d blocks of O^T
    static constexpr int ROWS = 16 * kRT * kGroups; // query rows per workgroup
    static constexpr int CPRL = ROWL / 16;          // 16-byte chunks per row
    static constexpr int RPI = 1024 / ROWL;         // key rows per LDS-direct load
    static constexpr int LROWS = kKT / 4;           // key rows a wave loads per tile
    static constexpr int LINS = LROWS / RPI;        // loads per wave per tile
    static_assert(LINS * RPI == LROWS, "a wave's rows fill whole loads");
};

// A loop phase known at compile time (the tile index mod 4 selects the K and
// V slots, so each slot is its own LDS array and the compiler can tell the
// tile loads in flight from the reads of another slot; mod 2 it selects the
// score wave's register set).
template <int N>
struct Ph {
    static constexpr int v = N;
};

template <int Q, class T>
__device__ __forceinline__ T& pick(T& a, T& b)
{
    if constexpr (Q == 0)
        return a;
    else
        return b;
}

template <int Q, class T>
__device__ __forceinline__ T& pick4(T& a, T& b, T& c, T& d)
{
    if constexpr (Q % 4 == 0)
        return a;
    else if constexpr (Q % 4 == 1)
        return b;
    else if constexpr (Q % 4 == 2)
        return c;
    else
        return d;
}

// Shared state of one workgroup besides the K and V slots.
template <int D, bool F8>
struct Smem {
    // P^T operands, by (tile parity, group, row tile, lane): bf16, or E4M3
    u32x4 p[2][kGroups][kRT][F8 ? 1 : 64];
    i32x2 p8[2][kGroups][kRT][F8 ? 64 : 1];
    float alpha[2][kGroups][kRT][16];  // rescale factor of each row
    int flag[2][kGroups];              // a group rescaled some rows in that tile
    float lsum[kGroups][kRT][16];      // row sums at the end
    float ksc[4][2], vsc[4][2];        // (F8) page scales of each K and V slot
    int vexp;                          // (F8) O is held divided by 2^vexp
    int bad;
};

struct Seq {
    int C;     // keys in the sequence (ctx_len)
    int kend;  // keys the workgroup loads: min(C, its tiles' end)
    int lo;    // first key any row of the workgroup attends (window / floor)
    int kh, Hk;
    int64_t n_pages;
    const __attribute__((address_space(4))) int32_t* bt;  // the sequence's block-table row
};

// Block-table entry of the page holding key0 .. key0 + 15 (0 past the
// workgroup's pages; prep_rows decides whether the page is read).  A scalar
// load: the vector memory path is left to the tile loads.
__device__ __forceinline__ int fetch_page(const Seq& b, int key0)
{
    const int k = __builtin_amdgcn_readfirstlane(key0);
    int v = 0;
    if (k < b.kend)
        v = b.bt[k >> 4];
    return v;
}

// The descriptor of this wave's 8 key rows of one tensor's tile (one page):
// it covers the page's rows below ctx_len, or no rows for a page the
// workgroup does not read (the loads are still issued and read zeros, so
// the count per iteration is fixed).  key0: the page's first key.
template <class G>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t prep_rows(const uint8_t* pool, const Seq& b,
                                                            int key0, int raw, int* bad)
{
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
    return __builtin_amdgcn_make_buffer_rsrc((void*)(pool + base), (short)0, rows * G::ROWL,
                                             kRsrcFlags);
}

// (fp8) The page scale of the same page for kv head b.kh, by the scalar
// unit: 0 for a page the workgroup does not read (or outside the pool), so a
// V page without rows adds nothing and stays out of a tile's scale exponent.
__device__ __forceinline__ float page_scale(const __attribute__((address_space(4))) float* sc,
                                            const Seq& b, int key0, int raw)
{
    const int p = __builtin_amdgcn_readfirstlane(raw);
    if (key0 < b.kend && key0 + 16 > b.lo && p >= 0 && (int64_t)p < b.n_pages)
        return sc[(int64_t)p * b.Hk + b.kh];
    return 0.f;
}

// Load instruction j of this wave's rows (RPI rows, 1 KiB), a buffer load
// that writes LDS directly.  dst: the page's first row in the tile's LDS
// buffer; prow: the wave's first row in the page (0 or 8).
template <class G>
__device__ __forceinline__ void issue_row(__amdgpu_buffer_rsrc_t rs, char* dst, int prow,
                                          const int (&loff)[G::LINS], int j)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (LDS void*)(dst + (prow + j * G::RPI) * G::ROWL), 16, loff[j], 0, 0, 0);
}

// All of this wave's rows of one tensor's tile (prologue).
template <class G>
__device__ __forceinline__ void load_rows(char* dst, const uint8_t* pool, const Seq& b, int key0,
                                          int prow, int raw, const int (&loff)[G::LINS], int* bad)
{
    const __amdgpu_buffer_rsrc_t rs = prep_rows<G>(pool, b, key0, raw, bad);
#pragma unroll
    for (int j = 0; j < G::LINS; ++j)
        issue_row<G>(rs, dst, prow, loff, j);
}

// Scheduling groups that spread an iteration's NL tile loads evenly among
// its NM matrix instructions (NM / NL matrix instructions, then one load,
// and so on), so the eight waves of a workgroup do not queue at the texture
// addresser at the same moment.  Instructions outside the groups (LDS
// reads, vector ALU) are scheduled freely around them.
template <int NL, int NM>
__device__ __forceinline__ void spread_loads()
{
#pragma unroll
    for (int j = 0; j < NL; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, NM / NL, 0);  // matrix instructions
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);        // one vector-memory read
    }
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

template <int D, bool F8>
__global__ __launch_bounds__(512, 2) void prefill_pipe_kernel(PrefillArgs a)
{
    using G = PGeo<D, F8>;
    // K and V of tiles t = 0, 1, 2 (mod 3), then the rest.
    __shared__ __attribute__((aligned(1024))) char s_k0[G::TILEB];
    __shared__ __attribute__((aligned(1024))) char s_k1[G::TILEB];
    __shared__ __attribute__((aligned(1024))) char s_k2[G::TILEB];
    __shared__ __attribute__((aligned(1024))) char s_k3[G::TILEB];
    __shared__ __attribute__((aligned(1024))) char s_v0[G::TILEB];
    __shared__ __attribute__((aligned(1024))) char s_v1[G::TILEB];
    __shared__ __attribute__((aligned(1024))) char s_v2[G::TILEB];
    __shared__ __attribute__((aligned(1024))) char s_v3[G::TILEB];
    __shared__ __attribute__((aligned(1024))) Smem<D, F8> sm;
    auto kslot = [&](auto ph) -> char* {
        constexpr int P = decltype(ph)::v % 4;
        return P == 0 ? s_k0 : P == 1 ? s_k1 : P == 2 ? s_k2 : s_k3;
    };
    auto vslot = [&](auto ph) -> char* {
        constexpr int P = decltype(ph)::v % 4;
        return P == 0 ? s_v0 : P == 1 ? s_v1 : P == 2 ? s_v2 : s_v3;
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
    b.bt = (const __attribute__((address_space(4))) int32_t*)bt;

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
    // rr, so the tile ends up swizzled.  Each wave issues G::LINS tile loads
    // per iteration (table entries are scalar loads); a tile's loads have two
    // iterations to land, so "all but the last two iterations' loads done"
    // is vmcnt <= 2 G::LINS.
    const int lpage = (wave >> 1) & 1, prow = 8 * (wave & 1);
    const int pr0 = 16 * lpage;  // the wave's page's first row in a tile
    const bool score = wave < 4;
    int loff[G::LINS];
    {
        const int rr = lane / G::CPRL, pc = lane % G::CPRL;
#pragma unroll
        for (int i = 0; i < G::LINS; ++i) {
            const int r = prow + i * G::RPI + rr;  // row in the page
            int sw = swz(r);
            if constexpr (F8)
                sw = score ? swzk<G::CPRL>(r) : swzv<G::CPRL>(pr0 + r);
            loff[i] = r * G::ROWL + ((pc ^ sw) * 16);
        }
    }
    constexpr int kInFlight = 2 * G::LINS;
    // (F8) page scales by the scalar unit; the wave loading a page's first
    // rows (prow 0) writes its scale beside the tile.
    const __attribute__((address_space(4))) float* ksp =
        (const __attribute__((address_space(4))) float*)a.k_scale;
    const __attribute__((address_space(4))) float* vsp =
        (const __attribute__((address_space(4))) float*)a.v_scale;
    auto put_scale = [&](float (&dst)[2], float sc) {
        if (lane == 0 && prow == 0)
            dst[lpage] = sc;
    };
    auto load_tile = [&](char* dst, const uint8_t* pool, bool isk, int slot, int key, int raw) {
        load_rows<G>(dst + pr0 * G::ROWL, pool, b, key, prow, raw, loff, &bad);
        if constexpr (F8)
            put_scale(isk ? sm.ksc[slot] : sm.vsc[slot], page_scale(isk ? ksp : vsp, b, key, raw));
    };

    // Prologue: K(0..3) (score waves) and V(0..2) (output waves), and the
    // table entries of the next two tiles each role loads (K(4), K(5);
    // V(3), V(4)), all landed.  (K(4) is loaded once the score waves have
    // read K(0).)
    const int k0 = ts * kKT + pr0;  // the wave's page's first key in tile ts
    int raw0, raw1;
    if (score) {
        load_tile(s_k0, kp, true, 0, k0, fetch_page(b, k0));
        load_tile(s_k1, kp, true, 1, k0 + kKT, fetch_page(b, k0 + kKT));
        load_tile(s_k2, kp, true, 2, k0 + 2 * kKT, fetch_page(b, k0 + 2 * kKT));
        load_tile(s_k3, kp, true, 3, k0 + 3 * kKT, fetch_page(b, k0 + 3 * kKT));
        raw0 = fetch_page(b, k0 + 4 * kKT);
        raw1 = fetch_page(b, k0 + 5 * kKT);
    } else {
        load_tile(s_v0, vp, false, 0, k0, fetch_page(b, k0));
        load_tile(s_v1, vp, false, 1, k0 + kKT, fetch_page(b, k0 + kKT));
        load_tile(s_v2, vp, false, 2, k0 + 2 * kKT, fetch_page(b, k0 + 2 * kKT));
        raw0 = fetch_page(b, k0 + 3 * kKT);
        raw1 = fetch_page(b, k0 + 4 * kKT);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    if (score) {
        // ---- score wave: Q^T in registers, K from LDS, softmax, P^T out.
        u32x4 qop[F8 ? 1 : kRT][F8 ? 1 : G::KSTEPS];  // Q^T operand: d = 32 st + 8 kb + 0..7
        i32x8 qf[F8 ? kRT : 1][F8 ? G::QS : 1];         // (F8) the same rounded to E4M3
        float qsc[kRT];                                  // (F8) its power-of-two scale
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
            const bool valid = row[rt] < n_rows;
            const uint16_t* q =
                (const uint16_t*)a.q + ((tok0 + (valid ? row[rt] : 0)) * H + head[rt]) * D;
            qsc[rt] = 1.f;
            if constexpr (F8) {
                qsc[rt] = qround::round_q<G::QS>(q, valid, kb, qf[rt]);
            } else {
#pragma unroll
                for (int st = 0; st < G::KSTEPS; ++st)
                    qop[rt][st] =
                        valid ? *(const u32x4*)(q + 32 * st + 8 * kb) : u32x4{0u, 0u, 0u, 0u};
            }
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
        const int skq = swzk<G::CPRL>(n);  // (F8) K rows 16 kq + n
        auto scores = [&](const char* ks, f32x4 (&s)[kRT][2]) {
            if constexpr (F8) {
                // k-step st: logical chunks 8 st + 2 kb and + 1 of key row
                // 16 kq + n (d = 128 st + 32 kb + 0..31).
#pragma unroll
                for (int kq = 0; kq < 2; ++kq) {
                    const char* kr = ks + (16 * kq + n) * G::ROWL;
                    i32x8 kw8[G::QS];
#pragma unroll
                    for (int st = 0; st < G::QS; ++st) {
                        const u32x4 c0 = *(const u32x4*)(kr + ((8 * st + 2 * kb) ^ skq) * 16);
                        const u32x4 c1 = *(const u32x4*)(kr + ((8 * st + 2 * kb + 1) ^ skq) * 16);
                        kw8[st] = i32x8{(int)c0[0], (int)c0[1], (int)c0[2], (int)c0[3],
                                        (int)c1[0], (int)c1[1], (int)c1[2], (int)c1[3]};
                    }
#pragma unroll
                    for (int rt = 0; rt < kRT; ++rt) {
                        s[rt][kq] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int st = 0; st < G::QS; ++st)
                            s[rt][kq] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                kw8[st], qf[rt][st], s[rt][kq], 0, 0, 0, 0, 0, 0);
                    }
                }
                return;
            }
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
        // Software pipeline, two tiles deep: iteration i computes the scores
        // of tile i + 2 on the matrix unit while tile i's softmax runs, so the
        // softmax never waits for products still queued in the matrix unit
        // behind the output wave's.  The scores of tile t live in s0..s3
        // (t mod 4).
        f32x4 s0[kRT][2], s1[kRT][2], s2[kRT][2], s3[kRT][2];
        // (F8) the K page scales of the tile in s0 .. s3, read with its scores
        float c0[2] = {1.f, 1.f}, c1[2] = {1.f, 1.f}, c2[2] = {1.f, 1.f}, c3[2] = {1.f, 1.f};
        auto kscales = [&](float (&c)[2], int slot) {
            if constexpr (F8) {
                c[0] = sm.ksc[slot][0];
                c[1] = sm.ksc[slot][1];
            }
        };
        int vexp = 0;  // (F8) O is held divided by 2^vexp
        scores(s_k0, s0);
        kscales(c0, 0);
        scores(s_k1, s1);
        kscales(c1, 1);
        // K(4) goes into K(0)'s slot: every score wave must have read K(0)
        // and K(1) first (the output waves take this barrier before their
        // loop).
        __syncthreads();
        load_tile(s_k0, kp, true, 0, k0 + 4 * kKT, raw0);
        raw0 = raw1;
        raw1 = fetch_page(b, k0 + 6 * kKT);
        // Iteration i, phase P = i mod 4.
        auto body = [&](int i, auto ph) {
            constexpr int P = decltype(ph)::v;
            auto& s = pick4<P>(s0, s1, s2, s3);       // tile i
            auto& sn = pick4<P + 2>(s0, s1, s2, s3);  // tile i + 2
            auto& kc = pick4<P>(c0, c1, c2, c3);
            auto& kcn = pick4<P + 2>(c0, c1, c2, c3);
            // K(i + 5) goes into the slot K(i + 1) held (read last in
            // iteration i - 1); its table entry was fetched two iterations ago,
            // the entry of K(i + 7) is fetched now.
            const __amdgpu_buffer_rsrc_t rl =
                prep_rows<G>(kp, b, k0 + (i + 5) * kKT, raw0, &bad);
            float ksc_new = 0.f;
            if constexpr (F8)
                ksc_new = page_scale(ksp, b, k0 + (i + 5) * kKT, raw0);
            char* kdst = kslot(Ph<P + 1>()) + pr0 * G::ROWL;
            raw0 = raw1;
            raw1 = fetch_page(b, k0 + (i + 7) * kKT);
            if (i < T) {
                const int buf = i & 1;
                const int tile0 = (ts + i) * kKT;
                // (F8) The scores of tile i + 2 first: their half-length
                // matrix work then starts before the softmax (measured 2%
                // faster; slower in the bf16 form, which issues them below).
                if constexpr (F8) {
                    scores(kslot(Ph<P + 2>()), sn);
                    kscales(kcn, (P + 2) % 4);
                }
                // Scale (log2 units); on a tile crossing the causal edge or a
                // row's first key, mask.  Then the lane-local max check.
                const bool diag = tile0 + kKT - 1 > minpos || tile0 < lo_max;
                // Factor of each score in the exponent: the softmax scale, and
                // with F8 the K page scale and the query's power of two.
                float sx[kRT][2];
#pragma unroll
                for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
                    for (int kq = 0; kq < 2; ++kq)
                        sx[rt][kq] = F8 ? kc[kq] * (sm_log2 * qsc[rt]) : sm_log2;
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
                                                    : s[rt][kq][x] * sx[rt][kq];
                                s[rt][kq][x] = v;
                                mx = fmaxf(mx, v);
                            }
                        lmax[rt] = mx;
#pragma unroll
                        for (int kq = 0; kq < 2; ++kq)
                            sx[rt][kq] = 1.f;
                    }
                } else {
#pragma unroll
                    for (int rt = 0; rt < kRT; ++rt) {
                        float mx = neg_inf();
                        if constexpr (F8) {
#pragma unroll
                            for (int kq = 0; kq < 2; ++kq)
                                mx = fmaxf(mx, fmaxf(fmaxf(s[rt][kq][0], s[rt][kq][1]),
                                                     fmaxf(s[rt][kq][2], s[rt][kq][3])) *
                                                   sx[rt][kq]);
                            lmax[rt] = mx;
                        } else {
#pragma unroll
                            for (int kq = 0; kq < 2; ++kq)
                                mx = fmaxf(mx, fmaxf(fmaxf(s[rt][kq][0], s[rt][kq][1]),
                                                     fmaxf(s[rt][kq][2], s[rt][kq][3])));
                            lmax[rt] = mx * sm_log2;
                        }
                    }
                }
                bool up = false;
#pragma unroll
                for (int rt = 0; rt < kRT; ++rt)
                    up = up || lmax[rt] > m[rt] + kTau;
                // (F8) The tile's V page scales join P before its E4M3 rounding
                // as vs / 2^F, F the exponent of the tile's largest scale (every
                // factor in (0, 1], so a probability keeps its E4M3 precision);
                // O is held divided by 2^F and moved exactly, through the rows'
                // rescale factors, when F changes.
                float fac[2] = {1.f, 1.f};
                float mv = 1.f;
                bool vch = false;
                if constexpr (F8) {
                    const float vs0 = sm.vsc[P % 4][0], vs1 = sm.vsc[P % 4][1];
                    const float vmax = fmaxf(vs0, vs1);
                    int f = vexp;
                    if (vmax > 0.f)
                        (void)__builtin_frexpf(vmax, &f);
                    if (f != vexp) {
                        mv = __builtin_ldexpf(1.f, vexp - f);
                        vexp = f;
                        vch = true;
                    }
                    fac[0] = __builtin_ldexpf(vs0, -vexp);
                    fac[1] = __builtin_ldexpf(vs1, -vexp);
                }
                const bool any = __builtin_amdgcn_ballot_w64(up) != 0 || vch;
                if (any) {
#pragma unroll
                    for (int rt = 0; rt < kRT; ++rt) {
                        const float mnew = fmaxf(m[rt], row_max4(lmax[rt]));
                        const float alpha =
                            m[rt] == neg_inf() ? 0.f : __builtin_amdgcn_exp2f(m[rt] - mnew);
                        l[rt] = l[rt] * alpha;
                        m[rt] = mnew;
                        if (kb == 0)
                            sm.alpha[buf][grp][rt][n] = F8 ? alpha * mv : alpha;
                    }
                }
                if (lane == 0)
                    sm.flag[buf][grp] = any ? 1 : 0;

                // The scores of tile i + 2 (stale K past the last tile: never
                // used), issued beside tile i's probabilities, this lane's part
                // of the row sums, and the P^T operand: k index j of the 32-key
                // step is key 16 (j / 4) + 4 kb + j % 4, matching the V^T reads.
                if constexpr (!F8)
                    scores(kslot(Ph<P + 2>()), sn);
#pragma unroll
                for (int rt = 0; rt < kRT; ++rt) {
                    const float mu = m[rt] == neg_inf() ? 0.f : m[rt];
                    float e[2][4];
#pragma unroll
                    for (int kq = 0; kq < 2; ++kq)
#pragma unroll
                        for (int x = 0; x < 4; ++x)
                            e[kq][x] = __builtin_amdgcn_exp2f(
                                __builtin_fmaf(s[rt][kq][x], sx[rt][kq], -mu));
                    l[rt] = l[rt] + (((e[0][0] + e[0][1]) + (e[0][2] + e[0][3])) +
                                     ((e[1][0] + e[1][1]) + (e[1][2] + e[1][3])));
                    if constexpr (F8) {
                        // P^T as E4M3 (nearest, ties to even): byte j is key
                        // 16 (j / 4) + 4 kb + j % 4, the key whose V the
                        // transposing read puts in byte j of the V^T operand.
                        int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(e[0][0] * fac[0],
                                                                 e[0][1] * fac[0], 0, false);
                        w0 = __builtin_amdgcn_cvt_pk_fp8_f32(e[0][2] * fac[0], e[0][3] * fac[0],
                                                             w0, true);
                        int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(e[1][0] * fac[1],
                                                                 e[1][1] * fac[1], 0, false);
                        w1 = __builtin_amdgcn_cvt_pk_fp8_f32(e[1][2] * fac[1], e[1][3] * fac[1],
                                                             w1, true);
                        sm.p8[buf][grp][rt][lane] = i32x2{w0, w1};
                    } else {
                        u32x4 pw;
                        pw[0] = pack_bf16(e[0][0], e[0][1]);
                        pw[1] = pack_bf16(e[0][2], e[0][3]);
                        pw[2] = pack_bf16(e[1][0], e[1][1]);
                        pw[3] = pack_bf16(e[1][2], e[1][3]);
                        sm.p[buf][grp][rt][lane] = pw;
                    }
                }
                // The tile loads, spread among the matrix instructions.
#pragma unroll
                for (int j = 0; j < G::LINS; ++j)
                    issue_row<G>(rl, kdst, prow, loff, j);
                spread_loads<G::LINS, F8 ? 4 * G::QS : 4 * G::KSTEPS>();
            } else {
#pragma unroll
                for (int j = 0; j < G::LINS; ++j)
                    issue_row<G>(rl, kdst, prow, loff, j);
            }
            if constexpr (F8)
                put_scale(sm.ksc[(P + 1) % 4], ksc_new);
            // K(i + 3) (issued in iteration i - 2) has landed; K(i + 4) and
            // K(i + 5) may still be in flight.
            tile_barrier<kInFlight>();
        };
        for (int i = 0; i <= T; i += 4) {
            body(i, Ph<0>());
            if (i + 1 <= T)
                body(i + 1, Ph<1>());
            if (i + 2 <= T)
                body(i + 2, Ph<2>());
            if (i + 3 <= T)
                body(i + 3, Ph<3>());
        }
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
            const float ls = row_sum4(l[rt]);
            if (kb == 0)
                sm.lsum[grp][rt][n] = ls;
        }
        if (F8 && wave == 0 && lane == 0)
            sm.vexp = vexp;
        if (bad)
            sm.bad = 1;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    } else {
        // ---- output wave: O^T += V^T . P^T, one tile behind, for 64 rows
        // (the row groups 2 rh and 2 rh + 1) and one half of head_dim (dh):
        // each V operand read feeds four 16-row tiles.
        const int ow = wave - 4, rh = ow >> 1, dh = ow & 1;
        constexpr int DH = G::DBLK / 2;  // d blocks of the half
        int voff[DH];
        // (F8) V^T reads (ds_read_b64_tr_b8): in each 16-lane group the
        // lanes' 8-byte chunks form 8 rows of 16 bytes (lanes 2r and 2r + 1)
        // and lane i receives byte i % 8 of the chunk of lane 2r + i / 8, for
        // r = 0 .. 7.  Lane L of group kb points at key row r = L / 2 of the
        // group's eight keys (4 kb + r, then 16 + 4 kb + r - 4), d-values
        // 16 jb + 8 (L % 2) .. + 7, so lane i gets V[key r][16 jb + i]: row i
        // of the V^T operand, keys in the P^T operand's byte order.
        int v8row = 0, v8sw = 0;
        const int v8half = 8 * (lane & 1);
        if constexpr (F8) {
            const int r = (lane & 15) >> 1;
            const int key = r < 4 ? 4 * kb + r : 16 + 4 * kb + (r - 4);
            v8row = key * G::ROWL;
            v8sw = swzv<G::CPRL>(key);
        }
        {
            const int vkey = 4 * kb + (n >> 2);
            const int sw = swz(vkey);
#pragma unroll
            for (int j = 0; j < DH; ++j) {
                const int jb = dh * DH + j;
                voff[j] = vkey * G::ROWL + 16 * ((2 * (jb & 7) + ((n & 3) >> 1)) ^ sw) +
                          (n & 1) * 8 + 256 * (jb >> 3);
            }
        }
        // Tile t of the wave: group 2 rh + t / 2, row tile t % 2.
        f32x4 O[2 * kRT][DH];
#pragma unroll
        for (int t = 0; t < 2 * kRT; ++t)
#pragma unroll
            for (int j = 0; j < DH; ++j)
                O[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        __syncthreads();  // the score waves' barrier after the tile-0 scores
        // Iteration i, phase P = i mod 4: the products of tile i - 1 with V
        // operands read in iteration i - 1 (va, ping-pong by parity), the V
        // operands of tile i read from slot P, and V(i + 3) loaded into slot
        // P + 3, which V(i - 1) left free.
        u32x4 vaA[F8 ? 1 : DH], vaB[F8 ? 1 : DH];
        i32x2 v8A[F8 ? DH : 1], v8B[F8 ? DH : 1];  // (F8) V^T operands, E4M3
        auto body = [&](int i, auto ph) {
            constexpr int P = decltype(ph)::v;
            auto& va = pick<(P + 1) % 2>(vaA, vaB);  // V(i - 1)
            auto& vn = pick<P % 2>(vaA, vaB);        // V(i)
            auto& va8 = pick<(P + 1) % 2>(v8A, v8B);
            auto& vn8 = pick<P % 2>(v8A, v8B);
            // V(i + 3)'s table entry was fetched two iterations ago, the entry
            // of V(i + 5) is fetched now.
            const __amdgpu_buffer_rsrc_t rl =
                prep_rows<G>(vp, b, k0 + (i + 3) * kKT, raw0, &bad);
            float vsc_new = 0.f;
            if constexpr (F8)
                vsc_new = page_scale(vsp, b, k0 + (i + 3) * kKT, raw0);
            char* vdst = vslot(Ph<P + 3>()) + pr0 * G::ROWL;
            raw0 = raw1;
            raw1 = fetch_page(b, k0 + (i + 5) * kKT);
            if (i >= 1) {
                const int buf = (i - 1) & 1;
                u32x4 pw[F8 ? 1 : 2 * kRT];
                i32x2 pw8[F8 ? 2 * kRT : 1];
#pragma unroll
                for (int t = 0; t < 2 * kRT; ++t) {
                    if constexpr (F8)
                        pw8[t] = sm.p8[buf][2 * rh + (t >> 1)][t & 1][lane];
                    else
                        pw[t] = sm.p[buf][2 * rh + (t >> 1)][t & 1][lane];
                }
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    if (sm.flag[buf][2 * rh + h]) {
#pragma unroll
                        for (int rt = 0; rt < kRT; ++rt) {
                            const float al = sm.alpha[buf][2 * rh + h][rt][n];
#pragma unroll
                            for (int j = 0; j < DH; ++j)
                                O[2 * h + rt][j] = O[2 * h + rt][j] * al;
                        }
                    }
                }
#pragma unroll
                for (int j = 0; j < DH; ++j)
#pragma unroll
                    for (int t = 0; t < 2 * kRT; ++t) {
                        if constexpr (F8)
                            O[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(
                                __builtin_bit_cast(long, va8[j]), __builtin_bit_cast(long, pw8[t]),
                                O[t][j], 0, 0, 0);
                        else
                            O[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8, va[j]),
                                __builtin_bit_cast(bf16x8, pw[t]), O[t][j], 0, 0, 0);
                    }
            }
            if (i < T) {
                const char* vr = vslot(Ph<P>());
                if constexpr (F8) {
#pragma unroll
                    for (int j = 0; j < DH; ++j)
                        vn8[j] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                            (LDS i32x2*)(vr + v8row + (((dh * DH + j) ^ v8sw) << 4) + v8half));
                } else {
#pragma unroll
                    for (int j = 0; j < DH; ++j) {
                        const char* v0 = vr + voff[j];
                        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS s16x4*)v0);
                        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (LDS s16x4*)(v0 + 16 * G::ROWL));
                        const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
                        const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
                        vn[j] = u32x4{l2[0], l2[1], h2[0], h2[1]};
                    }
                }
            }
            // The tile loads, spread among the matrix instructions.
#pragma unroll
            for (int j = 0; j < G::LINS; ++j)
                issue_row<G>(rl, vdst, prow, loff, j);
            if (i >= 1)
                spread_loads<G::LINS, 2 * kRT * DH>();
            if constexpr (F8)
                put_scale(sm.vsc[(P + 3) % 4], vsc_new);
            // V(i + 1) (issued in iteration i - 2) has landed; V(i + 2) and
            // V(i + 3) may still be in flight.
            tile_barrier<kInFlight>();
        };
        for (int i = 0; i <= T; i += 4) {
            body(i, Ph<0>());
            if (i + 1 <= T)
                body(i + 1, Ph<1>());
            if (i + 2 <= T)
                body(i + 2, Ph<2>());
            if (i + 3 <= T)
                body(i + 3, Ph<3>());
        }
        if (bad)
            sm.bad = 1;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        const bool nan = sm.bad != 0;
#pragma unroll
        for (int t = 0; t < 2 * kRT; ++t) {
            const int wrow = 16 * (2 * kRT * rh + t) + n;  // row in the workgroup
            const int hg = wrow / BP, p = wrow - hg * BP;
            const int r = pb * BP + p;
            if (r >= n_rows)
                continue;
            const int hd = kh * g + hg;
            const float ls = sm.lsum[2 * rh + (t >> 1)][t & 1][n];
            const float inv = F8 ? __builtin_ldexpf(1.f / ls, sm.vexp) : 1.f / ls;
            uint16_t* out = (uint16_t*)a.out + ((tok0 + r) * H + hd) * D;
#pragma unroll
            for (int j = 0; j < DH; ++j) {
                const int d = 16 * (dh * DH + j) + 4 * kb;
                u32x2 o;
                o[0] = nan ? 0x7FC07FC0u : pack_bf16(O[t][j][0] * inv, O[t][j][1] * inv);
                o[1] = nan ? 0x7FC07FC0u : pack_bf16(O[t][j][2] * inv, O[t][j][3] * inv);
                *(u32x2*)(out + d) = o;
            }
        }
    }
}

template <int D, bool F8>
hipError_t launch_d(const PrefillArgs& a, hipStream_t stream)
{
    using G = PGeo<D, F8>;
    const int g = a.n_head / a.n_head_kv;
    const int BP = G::ROWS / g;
    const int npbm = ((a.cu_seqlens ? a.max_q_len : a.n_rows) + BP - 1) / BP;
    const int64_t nblk = (int64_t)(a.cu_seqlens ? a.n_var : 1) * npbm * a.n_head_kv;
    if (nblk > (int64_t)1 << 30)
        return hipErrorInvalidValue;
    const int grid = (int)((nblk + 7) / 8) * 8;
    if (a.ev_start)
        (void)hipEventRecord(a.ev_start, stream);
    hipLaunchKernelGGL((prefill_pipe_kernel<D, F8>), dim3(grid), dim3(512), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && a.ev_stop)
        (void)hipEventRecord(a.ev_stop, stream);
    return e;
}

}  // namespace

// bf16 cache, or fp8 cache with both fp8 bits (QK^T and PV on the fp8
// matrix unit); head_dim 128 or 256, g a divisor of 128.  Other shapes are
// refused (hipErrorNotSupported) and take the one-role kernel.
hipError_t launch_prefill_pipe(const PrefillArgs& a, hipStream_t stream)
{
    const int g = a.n_head / a.n_head_kv;
    if (g > 128 || 128 % g != 0)
        return hipErrorNotSupported;
    const bool f8 = a.fp8 && a.qk_fp8 && a.pv_fp8;
    if (!f8 && (a.fp8 || a.qk_fp8 || a.pv_fp8))
        return hipErrorNotSupported;
    if (a.head_dim == 128)
        return f8 ? launch_d<128, true>(a, stream) : launch_d<128, false>(a, stream);
    if (a.head_dim == 256)
        return f8 ? launch_d<256, true>(a, stream) : launch_d<256, false>(a, stream);
    return hipErrorNotSupported;
}

}  // namespace pa
