// prefill.hip -- a chunk of new rows of ONE sequence over its paged cache
// ("kern manifest v7" schema, $defs.Batch: one sequence, as many rows as the
// chunk; `context` is the cached rows the call expands over).  Row r of an
// n_rows chunk sits at position ctx_len - n_rows + r and attends to keys
// 0 .. that position.
//
// Work decomposition (gfx950)
//   A workgroup of NW waves owns one kv head and 16 RT NW query rows:
//   that many rows / g consecutive positions x the g query heads sharing the
//   kv head, so every K/V tile it stages serves g heads.  Wave w owns RT
//   16-row tiles (rows 16 (RT w + rt) + 0..15); each K or V operand read from
//   LDS feeds RT matrix instructions.
//   Keys stream in 64-key tiles (four 16-token pages).  K and V tiles live in
//   two LDS buffers each, row-major as bf16 with each row's 16-byte chunks
//   XOR-swizzled by the row index (conflict-free reads of a column of rows).
//   bf16 pages are copied global -> LDS by buffer loads that write LDS
//   directly (no registers in flight); the buffer descriptor of each page
//   covers only the rows below ctx_len, so rows past the context arrive as
//   zeros.  fp8 pages are loaded into registers, converted to bf16 exactly
//   and written to the same layout.
//   Software pipeline: the scores of tile t+1 are computed while tile t's
//   softmax runs, so the matrix unit has independent work during the
//   exponentials.  Iteration t therefore reads K(t+1) and V(t) and fills
//   K(t+2) and V(t+1) into the buffers K(t) and V(t-1) left free.
//   Per wave and tile, on v_mfma_f32_16x16x32_bf16:
//     S^T[key][row] = K . Q^T      K rows by ds_read_b128, Q^T in registers
//     online softmax               a row's 16 scores of the tile sit in the 4
//                                  lanes row + 16 j; each lane keeps its own
//                                  part of the row sum, and the row max is
//                                  only gathered across the 4 lanes when a
//                                  lane's score exceeds it by more than 2^8
//                                  (checked once per tile, before any score of
//                                  the tile becomes a probability)
//     O^T[d][row]  += V^T . P^T    V^T by ds_read_b64_tr_b16 (a 4-key x
//                                  16-column block per 16 lanes, transposed
//                                  in the read); P^T is the S^T accumulator
//                                  re-packed in place; O^T's row is again
//                                  the lane's row, so rescaling and 1/l are
//                                  lane-local
//   Workgroups of one kv head are placed on the same XCDs (blockIdx mod 8
//   picks the XCD) so the K/V tiles they stream share that XCD's L2.
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
constexpr int kKT = 64;       // keys per tile
constexpr float kTau = 8.f;   // lazy-rescale threshold (log2 units)
constexpr int kRsrcFlags = 0x00020000;

__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }

// Two floats to a bf16 pair (round to nearest even), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
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

// Physical 16-byte chunk of logical chunk c of an fp8 K row (CK chunks)
// in LDS row r is c ^ swzk<CK>(r).  The QK^T operand reads take one chunk
// of each of 16 consecutive rows: for 256-byte rows (a full bank line each)
// swzk is one-to-one on r mod 16; for 128-byte rows (two to a bank line) it
// is one-to-one on r / 2 mod 8, so the 8 rows sharing a half of the banks
// hit different chunks.
template <int CK>
__device__ __forceinline__ int swzk(int r)
{
    return CK == 16 ? (r & 15) : ((r >> 1) & 7);
}

template <int D, bool FP8, int RT, int NW>
struct PGeo {
    static constexpr int NTH = 64 * NW;          // threads per workgroup
    static constexpr int ROWS = 16 * RT * NW;    // query rows per workgroup
    static constexpr int EB = FP8 ? 1 : 2;
    static constexpr int ROWB = D * EB;          // bytes of one token row in the pool
    static constexpr int ROWL = D * 2;           // bytes of one row in LDS (bf16)
    static constexpr int CPRL = ROWL / 16;       // 16-byte chunks per LDS row
    static constexpr int TILEB = kKT * ROWL;     // one K (or V) tile in LDS
    static constexpr int KSTEPS = D / 32;        // k-steps of QK^T
    static constexpr int DBLK = D / 16;          // 16-wide d blocks of O^T
    // direct (bf16) loads: 1 KiB LDS blocks
    static constexpr int RPB = 1024 / ROWL;            // rows per block
    static constexpr int NBW = (kKT / RPB) / NW;       // blocks per wave per tensor
    // Each wave loads KPW consecutive keys of a tile, all in one page.
    static constexpr int KPW = kKT / NW;
    // staged (fp8) loads: 16-byte pool chunks per lane per tensor
    static constexpr int CPR = ROWB / 16;
    static constexpr int SCH = KPW * CPR / 64;
    static_assert(NBW * RPB == KPW && KPW <= 16, "direct loads: one page per wave");
    static_assert(SCH * 64 == KPW * CPR, "staged loads must cover the wave's keys");
};

struct Blk {
    int C, kh, Hk;
    int lo;  // first key any row of the workgroup attends (window / floor)
    int64_t n_pages;
    const int32_t* bt;
};

// Block-table entry of the page holding keys key0 .. key0 + 15 (raw, not yet
// checked); -1 past the context and for a page wholly below the first key
// attended (a runtime floor may have released it).  Issued tiles ahead so
// its latency hides behind compute.
__device__ __forceinline__ int fetch_page(const Blk& b, int key0)
{
    return key0 < b.C && key0 + 16 > b.lo ? b.bt[key0 >> 4] : -1;
}

// That page and the number of its rows below the context; page -1 (and 0
// rows) past the context or for an entry outside the pool (which also raises
// *bad).
__device__ __forceinline__ void resolve_page(const Blk& b, int key0, int raw, int& pg, int& rows,
                                             int* bad)
{
    const int p = __builtin_amdgcn_readfirstlane(raw);
    pg = -1;
    rows = 0;
    if (key0 < b.C && key0 + 16 > b.lo) {
        if (p < 0 || (int64_t)p >= b.n_pages) {
            *bad = 1;
        } else {
            pg = p;
            rows = min(16, b.C - key0);
        }
    }
}

// bf16: this wave's KPW keys of one tensor's tile (one page), as buffer
// loads that write LDS directly.  key0 is the page's first key.
template <class G>
__device__ __forceinline__ void issue_direct(char* dst, const uint8_t* pool, const Blk& b,
                                             int key0, int wave, const int (&loff)[G::NBW],
                                             int raw, int* bad)
{
    int pg, rows;
    resolve_page(b, key0, raw, pg, rows, bad);
    const int64_t base = ((int64_t)(pg < 0 ? 0 : pg) * b.Hk + b.kh) * 16 * G::ROWB;
    __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(pool + base), (short)0, rows * G::ROWB, kRsrcFlags);
#pragma unroll
    for (int i = 0; i < G::NBW; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (LDS void*)(dst + (wave * G::NBW + i) * 1024), 16, loff[i], 0, 0, 0);
}

// fp8: a lane's share of the wave's KPW keys of one tensor's tile in
// registers between load and store, with the page's scale.
template <class G>
struct Staged {
    u32x4 c[G::SCH];
    float s;
};

template <class G>
__device__ __forceinline__ void stage_load(Staged<G>& st, const uint8_t* pool, const float* scl,
                                           const Blk& b, int key0, int wave, int lane, int raw,
                                           int* bad, float none = 1.f)
{
    int pg, rows;
    resolve_page(b, key0, raw, pg, rows, bad);
#pragma unroll
    for (int i = 0; i < G::SCH; ++i) {
        const int c = i * 64 + lane;
        const int pr = ((wave * G::KPW) & 15) + c / G::CPR, piece = c % G::CPR;  // page row
        if (pr < rows) {
            const int64_t off =
                (((int64_t)pg * b.Hk + b.kh) * 16 + pr) * G::ROWB + piece * 16;
            st.c[i] = *(const u32x4*)(pool + off);
        } else {
            st.c[i] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    // A page past the context gets scale `none` (its keys are masked).
    if constexpr (G::EB == 1)
        st.s = pg >= 0 ? scl[(int64_t)pg * b.Hk + b.kh] : none;
    else
        st.s = 1.f;
}

// fp8 K kept as codes (QK^T on the fp8 matrix unit): rows of D bytes in
// LDS, chunks swizzled by swzk.
template <class G>
__device__ __forceinline__ void stage_store_codes(const Staged<G>& st, char* buf, float* sc,
                                                  int wave, int lane)
{
#pragma unroll
    for (int i = 0; i < G::SCH; ++i) {
        const int c = i * 64 + lane;
        const int key = wave * G::KPW + c / G::CPR, piece = c % G::CPR;
        *(u32x4*)(buf + key * G::ROWB + (piece ^ swzk<G::CPR>(key)) * 16) = st.c[i];
    }
    if (lane == 0 && ((wave * G::KPW) & 15) == 0)
        sc[(wave * G::KPW) >> 4] = st.s;
}

// fp8 V kept as codes (PV on the fp8 matrix unit): rows of D bytes, 16-byte
// chunks swizzled by swzv, which keeps the 8 rows one transposing read
// gathers (keys 4 kb .. 4 kb + 3 and 16 + the same of a 32-key half) on
// distinct chunk positions.
template <int CPR>
__device__ __forceinline__ int swzv(int key)
{
    return (key ^ (key >> 4)) & (CPR - 1);
}

template <class G>
__device__ __forceinline__ void stage_store_codes_v(const Staged<G>& st, char* buf, float* sc,
                                                    int wave, int lane)
{
#pragma unroll
    for (int i = 0; i < G::SCH; ++i) {
        const int c = i * 64 + lane;
        const int key = wave * G::KPW + c / G::CPR, piece = c % G::CPR;
        *(u32x4*)(buf + key * G::ROWB + (piece ^ swzv<G::CPR>(key)) * 16) = st.c[i];
    }
    if (lane == 0 && ((wave * G::KPW) & 15) == 0)
        sc[(wave * G::KPW) >> 4] = st.s;
}

template <class G>
__device__ __forceinline__ void stage_store(const Staged<G>& st, char* buf, float* sc, int wave,
                                            int lane)
{
#pragma unroll
    for (int i = 0; i < G::SCH; ++i) {
        const int c = i * 64 + lane;
        const int key = wave * G::KPW + c / G::CPR, piece = c % G::CPR;
        const u32x4 w = st.c[i];
        char* row = buf + key * G::ROWL;
        if constexpr (G::EB == 2) {  // bf16: stored as loaded
            *(u32x4*)(row + (piece ^ swz(key)) * 16) = w;
            continue;
        }
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
    if (lane == 0 && ((wave * G::KPW) & 15) == 0)
        sc[(wave * G::KPW) >> 4] = st.s;
}

// Max over the 4 lanes n, n + 16, n + 32, n + 48 (the lanes of one row).
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

template <int D, bool FP8, int RT, int NW, bool QF8, bool PV8>
__global__ __launch_bounds__(64 * NW, 2) void prefill_kernel(PrefillArgs a)
{
    using G = PGeo<D, FP8, RT, NW>;
    static_assert(!QF8 || (FP8 && RT == 1), "fp8 QK^T: fp8 cache, one row tile per wave");
    static_assert(!PV8 || (FP8 && RT == 1), "fp8 PV: fp8 cache, one row tile per wave");
    constexpr int QS = D / 128;  // k-steps of the fp8 QK^T (128 d-values each)
    constexpr bool STG = FP8;  // staged through registers (fp8) or LDS-direct (bf16)
    __shared__ __attribute__((aligned(1024))) char s_k0[G::TILEB];
    __shared__ __attribute__((aligned(1024))) char s_k1[G::TILEB];
    __shared__ __attribute__((aligned(1024))) char s_v0[G::TILEB];
    __shared__ __attribute__((aligned(1024))) char s_v1[G::TILEB];
    __shared__ float s_ksc[2][4], s_vsc[2][4];  // fp8 page scales of each buffer
    __shared__ int s_bad;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
    const int n = lane & 15, kb = lane >> 4;
    const int Hk = a.n_head_kv, H = a.n_head, g = H / Hk, BP = G::ROWS / g;
    // The workgroup's sequence: its rows, keys, first token row and table.
    int n_rows = a.n_rows, ctx_len = a.ctx_len;
    int64_t tok0 = 0;
    const int32_t* bt = a.block_table;
    // Blocks per sequence: position blocks (of the longest sequence) x kv heads.
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

    Blk b;
    b.C = ctx_len;
    b.kh = kh;
    b.Hk = Hk;
    b.n_pages = a.n_pages;
    b.bt = bt;
    const int base_pos = ctx_len - n_rows;
    const int rlast = min(n_rows, (pb + 1) * BP) - 1;
    const int maxpos = base_pos + rlast;  // last key any row here needs
    const int minpos = base_pos + pb * BP;
    const int nt = (maxpos + kKT) / kKT;
    // First key a row at position p attends: its sliding window and the
    // sequence's floor, whichever is later.
    auto key_floor = [&](int p) { return max(a.kv_floor, a.window > 0 ? p - a.window + 1 : 0); };
    const int lo_min = key_floor(minpos), lo_max = key_floor(maxpos);
    b.lo = lo_min;
    const int ts = lo_min / kKT;  // first tile with a key to attend

    // The lane's query row in each of the wave's row tiles (row n of 16).
    int row[RT], head[RT], pos[RT], klo[RT];
    u32x4 qop[RT][G::KSTEPS];  // Q^T operand: d = 32 st + 8 kb + 0..7
    // fp8 Q^T operand: byte i of k-step st is d = 128 st + 32 kb + i, the
    // query rounded to E4M3 at the power-of-two scale qsc of its vector.
    i32x8 qf[RT][QS];
    float qsc[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int wrow = 16 * (RT * wave + rt) + n;  // row in the workgroup
        const int hg = wrow / BP, p = wrow - hg * BP;
        row[rt] = pb * BP + p;
        head[rt] = kh * g + hg;
        const bool valid = row[rt] < n_rows;
        pos[rt] = valid ? base_pos + row[rt] : -1;
        klo[rt] = key_floor(pos[rt]);
        const uint16_t* q =
            (const uint16_t*)a.q + ((tok0 + (valid ? row[rt] : 0)) * H + head[rt]) * D;
        qsc[rt] = 1.f;
        if constexpr (QF8) {
            qsc[rt] = qround::round_q<QS>(q, valid, kb, qf[rt]);
        } else {
#pragma unroll
            for (int st = 0; st < G::KSTEPS; ++st)
                qop[rt][st] =
                    valid ? *(const u32x4*)(q + 32 * st + 8 * kb) : u32x4{0u, 0u, 0u, 0u};
        }
    }

    f32x4 O[RT][G::DBLK];
    float m[RT], l[RT];  // l: this lane's part of the row sum
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
        for (int jb = 0; jb < G::DBLK; ++jb)
            O[rt][jb] = f32x4{0.f, 0.f, 0.f, 0.f};
        m[rt] = neg_inf();
        l[rt] = 0.f;
    }
    int vexp = 0;  // (PV8) O is held divided by 2^vexp
    const float sm_log2 = kLog2e / __builtin_sqrtf((float)D);
    // Score factor of an fp8 page (times its K scale): with fp8 QK^T the
    // query's power-of-two scale too (exact).
    const float smq = QF8 ? sm_log2 * qsc[0] : sm_log2;

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
            const int r = (wave * G::NBW + i) * G::RPB + rr;
            loff[i] = (r & 15) * G::ROWB + ((pc ^ swz(r)) * 16);
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

    // PV8 V^T reads (ds_read_b64_tr_b8): in each 16-lane group the lanes'
    // 8-byte chunks form 8 rows of 16 bytes (lanes 2r and 2r + 1) and lane i
    // receives byte i % 8 of the chunk of lane 2r + i / 8 for r = 0 .. 7.
    // Lane L of group kb points at key row r = L / 2 of its group's eight
    // keys (4 kb + r, then 16 + 4 kb + r - 4, in each 32-key half), d-values
    // 16 jb + 8 (L % 2) .. + 7, so lane i gets V[key r][16 jb + i] for r = 0
    // .. 7: row i of the V^T operand, keys in the P^T operand's order.
    int v8row[2] = {0, 0}, v8sw[2] = {0, 0};
    const int v8half = 8 * (lane & 1);
    if constexpr (PV8) {
        const int r = (lane & 15) >> 1;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int key = 32 * hf + (r < 4 ? 4 * kb + r : 16 + 4 * kb + (r - 4));
            v8row[hf] = key * G::ROWB;
            v8sw[hf] = swzv<G::CPR>(key);
        }
    }

    // S^T of a tile: [row tile][16-key block]; two sets, current and next.
    f32x4 sa[RT][4], sb[RT][4];
    float ka[4], kb4[4];  // K page scales (fp8) of the tile in sa / sb
    const int skq = swzk<G::CPR>(n);  // fp8 K rows: 16 kq + n, swizzle of n
    auto scores = [&](const char* ks, f32x4 (&acc)[RT][4], int kq) {
        if constexpr (QF8) {
            // K codes of key row 16 kq + n: k-step st is logical chunks
            // 8 st + 2 kb and + 1 (d = 128 st + 32 kb + 0..31).
            const char* kr = ks + (16 * kq + n) * G::ROWB;
            i32x8 kw8[QS];
#pragma unroll
            for (int st = 0; st < QS; ++st) {
                const u32x4 c0 = *(const u32x4*)(kr + ((8 * st + 2 * kb) ^ skq) * 16);
                const u32x4 c1 = *(const u32x4*)(kr + ((8 * st + 2 * kb + 1) ^ skq) * 16);
                kw8[st] = i32x8{(int)c0[0], (int)c0[1], (int)c0[2], (int)c0[3],
                                (int)c1[0], (int)c1[1], (int)c1[2], (int)c1[3]};
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                acc[rt][kq] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int st = 0; st < QS; ++st)
                    acc[rt][kq] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        kw8[st], qf[rt][st], acc[rt][kq], 0, 0, 0, 0, 0, 0);
            }
            return;
        }
        u32x4 kw[G::KSTEPS];
#pragma unroll
        for (int st = 0; st < G::KSTEPS; ++st)
            kw[st] = *(const u32x4*)(ks + koff[st % KBS] + kq * 16 * G::ROWL + 256 * (st / KBS));
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            acc[rt][kq] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < G::KSTEPS; ++st)
                acc[rt][kq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, kw[st]), __builtin_bit_cast(bf16x8, qop[rt][st]),
                    acc[rt][kq], 0, 0, 0);
        }
    };

    // The wave loads keys wave * KPW .. + KPW - 1 of every tile: one page,
    // whose first key is tile0 + wk.
    const int wk = ((wave * G::KPW) >> 4) * 16;
    Staged<G> stk, stv;
    // PV8: V stays as codes; a page with no rows gets V scale 0, so it does
    // not enter a tile's scale exponent below.
    constexpr float kNoV = PV8 ? 0.f : 1.f;
    auto store_v = [&](char* buf, float* sc) {
        if constexpr (PV8)
            stage_store_codes_v<G>(stv, buf, sc, wave, lane);
        else
            stage_store<G>(stv, buf, sc, wave, lane);
    };
    auto store_k = [&](char* buf, float* sc) {
        if constexpr (QF8)
            stage_store_codes<G>(stk, buf, sc, wave, lane);
        else
            stage_store<G>(stk, buf, sc, wave, lane);
    };
    const int k0 = ts * kKT;
    int rawv = fetch_page(b, k0 + wk);        // block-table entries of the next V
    int rawk = fetch_page(b, k0 + kKT + wk);  // and K tiles to load
    if constexpr (STG) {
        stage_load<G>(stk, kp, a.k_scale, b, k0 + wk, wave, lane, rawv, &bad);
        store_k(s_k0, s_ksc[0]);
        stage_load<G>(stv, vp, a.v_scale, b, k0 + wk, wave, lane, rawv, &bad, kNoV);
        store_v(s_v0, s_vsc[0]);
        if (nt > ts + 1) {
            stage_load<G>(stk, kp, a.k_scale, b, k0 + kKT + wk, wave, lane, rawk, &bad);
            store_k(s_k1, s_ksc[1]);
        }
    } else {
        issue_direct<G>(s_k0, kp, b, k0 + wk, wave, loff, rawv, &bad);
        issue_direct<G>(s_v0, vp, b, k0 + wk, wave, loff, rawv, &bad);
        if (nt > ts + 1)
            issue_direct<G>(s_k1, kp, b, k0 + kKT + wk, wave, loff, rawk, &bad);
    }
    rawv = rawk;
    rawk = fetch_page(b, k0 + 2 * kKT + wk);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) {
        scores(s_k0, sa, kq);
        ka[kq] = FP8 ? s_ksc[0][kq] : 1.f;
    }

    // Iteration t: K(t+1) in kr, V(t) in vr; fills K(t+2) into kw and V(t+1)
    // into vw.  cur holds S^T(t) (kc its K scales); nxt receives S^T(t+1).
    auto tile_body = [&](int t, const char* kr, const char* vr, char* kwb, char* vwb,
                         const float* krs, const float* vrs, float* kws, float* vws,
                         f32x4 (&cur)[RT][4], const float (&kc)[4], f32x4 (&nxt)[RT][4],
                         float (&kn)[4]) {
        const int tile0 = t * kKT;
        if (t + 1 < nt) {
            if constexpr (STG)
                stage_load<G>(stv, vp, a.v_scale, b, tile0 + kKT + wk, wave, lane, rawv, &bad,
                              kNoV);
            else
                issue_direct<G>(vwb, vp, b, tile0 + kKT + wk, wave, loff, rawv, &bad);
        }
        if (t + 2 < nt) {
            if constexpr (STG)
                stage_load<G>(stk, kp, a.k_scale, b, tile0 + 2 * kKT + wk, wave, lane, rawk,
                              &bad);
            else
                issue_direct<G>(kwb, kp, b, tile0 + 2 * kKT + wk, wave, loff, rawk, &bad);
        }
        rawv = rawk;
        rawk = fetch_page(b, tile0 + 3 * kKT + wk);

        // On a tile that crosses the causal edge or the first key of some
        // row, mask (-inf); then each lane's max of its scaled scores.  The
        // scale is applied inside the exponent below either way, so whether
        // the workgroup counts a tile as crossing changes no row's bits.
        const bool diag = tile0 + kKT - 1 > minpos || tile0 < lo_max;
        float sx[4];  // factor applied to cur in the exponent
#pragma unroll
        for (int kq = 0; kq < 4; ++kq)
            sx[kq] = FP8 ? kc[kq] * smq : sm_log2;
        if (diag) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int kq = 0; kq < 4; ++kq)
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        const int key = tile0 + 16 * kq + 4 * kb + x;
                        if (key > pos[rt] || key < klo[rt])
                            cur[rt][kq][x] = neg_inf();
                    }
        }
        float lmax[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            float mx = neg_inf();
#pragma unroll
            for (int kq = 0; kq < 4; ++kq) {
                const float bm = fmaxf(fmaxf(cur[rt][kq][0], cur[rt][kq][1]),
                                       fmaxf(cur[rt][kq][2], cur[rt][kq][3]));
                mx = FP8 ? fmaxf(mx, bm * sx[kq]) : fmaxf(mx, bm);
            }
            lmax[rt] = FP8 ? mx : mx * sm_log2;
        }
        // Lazy rescale, decided per row: a row moves its max only when a
        // tile's max passes it by more than kTau, so a row's arithmetic never
        // depends on the other rows of its wave (or on the workgroup's size).
        bool up = false;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
            up = up || lmax[rt] > m[rt] + kTau;
        if (__builtin_amdgcn_ballot_w64(up)) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const float rm = row_max4(lmax[rt]);
                const bool need = rm > m[rt] + kTau;
                const float alpha =
                    !need ? 1.f : m[rt] == neg_inf() ? 0.f : __builtin_amdgcn_exp2f(m[rt] - rm);
                l[rt] = l[rt] * alpha;
#pragma unroll
                for (int jb = 0; jb < G::DBLK; ++jb)
                    O[rt][jb] = O[rt][jb] * alpha;
                m[rt] = need ? rm : m[rt];
            }
        }

        // PV8: the tile's V page scales join P before its E4M3 rounding as
        // vs / 2^F, F the exponent of the tile's largest scale (so every
        // factor lies in (0, 1] and a probability keeps its E4M3 precision);
        // O is held divided by 2^F and moved exactly when F changes.
        float fac[4];
        if constexpr (PV8) {
            const float vmax = fmaxf(fmaxf(vrs[0], vrs[1]), fmaxf(vrs[2], vrs[3]));
            int f = vexp;
            if (vmax > 0.f)
                (void)__builtin_frexpf(vmax, &f);
            if (f != vexp) {
                const float mv = __builtin_ldexpf(1.f, vexp - f);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int jb = 0; jb < G::DBLK; ++jb)
                        O[rt][jb] = O[rt][jb] * mv;
                vexp = f;
            }
#pragma unroll
            for (int kq = 0; kq < 4; ++kq)
                fac[kq] = __builtin_ldexpf(vrs[kq], -vexp);
        }

        // Scores of tile t+1 (on stale K past the last tile: never used),
        // interleaved with tile t's probabilities.
        float muse[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
            muse[rt] = m[rt] == neg_inf() ? 0.f : m[rt];
        float e[RT][4][4];
#pragma unroll
        for (int kq = 0; kq < 4; ++kq) {
            scores(kr, nxt, kq);
            kn[kq] = FP8 ? krs[kq] : 1.f;
            const float vsc = PV8 ? fac[kq] : FP8 ? vrs[kq] : 1.f;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                float pe[4];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    // (a masked key stays -inf whatever the page scale, 0 included)
                    const float c = cur[rt][kq][x];
                    pe[x] = __builtin_amdgcn_exp2f(
                        c == neg_inf() ? neg_inf() : __builtin_fmaf(c, sx[kq], -muse[rt]));
                    e[rt][kq][x] = FP8 ? pe[x] * vsc : pe[x];
                }
                l[rt] = l[rt] + ((pe[0] + pe[1]) + (pe[2] + pe[3]));
            }
        }
        if constexpr (PV8) {
            // P^T as E4M3 (nearest, ties to even): byte j of the 32-key half
            // hf is key 32 hf + 16 (j / 4) + 4 kb + j % 4, the key whose V
            // the transposing read puts in byte j of the V^T operand.
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                i32x2 p8[RT];
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(e[rt][2 * hf][0], e[rt][2 * hf][1], 0,
                                                             false);
                    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(e[rt][2 * hf][2], e[rt][2 * hf][3], w0,
                                                         true);
                    int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(e[rt][2 * hf + 1][0],
                                                             e[rt][2 * hf + 1][1], 0, false);
                    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(e[rt][2 * hf + 1][2],
                                                         e[rt][2 * hf + 1][3], w1, true);
                    p8[rt] = i32x2{w0, w1};
                }
                constexpr int NB = 4;  // d blocks per batch of V reads
#pragma unroll
                for (int j0 = 0; j0 < G::DBLK; j0 += NB) {
                    i32x2 va[NB];
#pragma unroll
                    for (int jj = 0; jj < NB; ++jj) {
                        const int jb = j0 + jj;
                        va[jj] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                            (LDS i32x2*)(vr + v8row[hf] + ((jb ^ v8sw[hf]) << 4) + v8half));
                    }
#pragma unroll
                    for (int jj = 0; jj < NB; ++jj)
#pragma unroll
                        for (int rt = 0; rt < RT; ++rt)
                            O[rt][j0 + jj] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(
                                __builtin_bit_cast(long, va[jj]), __builtin_bit_cast(long, p8[rt]),
                                O[rt][j0 + jj], 0, 0, 0);
                }
            }
        } else {
        // P^T operands: k index i of the 32-key half hf is key
        // 32 hf + 16 (i / 4) + 4 kb + i % 4, matching the V^T reads.
        u32x4 pb[RT][2];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                pb[rt][hf][0] = pack_bf16(e[rt][2 * hf][0], e[rt][2 * hf][1]);
                pb[rt][hf][1] = pack_bf16(e[rt][2 * hf][2], e[rt][2 * hf][3]);
                pb[rt][hf][2] = pack_bf16(e[rt][2 * hf + 1][0], e[rt][2 * hf + 1][1]);
                pb[rt][hf][3] = pack_bf16(e[rt][2 * hf + 1][2], e[rt][2 * hf + 1][3]);
            }

        // O^T += V^T . P^T, one 32-key k-step per half and d block.
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            constexpr int NB = 4;  // d blocks per batch of V reads
#pragma unroll
            for (int j0 = 0; j0 < G::DBLK; j0 += NB) {
                u32x4 va[NB];
#pragma unroll
                for (int jj = 0; jj < NB; ++jj) {
                    const int jb = j0 + jj;
                    const char* v0 = vr + voff[jb % VBS] + 32 * hf * G::ROWL + 256 * (jb / VBS);
                    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS s16x4*)v0);
                    const s16x4 hi =
                        __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS s16x4*)(v0 + 16 * G::ROWL));
                    const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
                    const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
                    va[jj] = u32x4{l2[0], l2[1], h2[0], h2[1]};
                }
#pragma unroll
                for (int jj = 0; jj < NB; ++jj)
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt)
                        O[rt][j0 + jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, va[jj]),
                            __builtin_bit_cast(bf16x8, pb[rt][hf]), O[rt][j0 + jj], 0, 0, 0);
            }
        }
        }

        if constexpr (STG) {
            if (t + 1 < nt)
                store_v(vwb, vws);
            if (t + 2 < nt)
                store_k(kwb, kws);
        } else {
            __builtin_amdgcn_s_waitcnt(0);
        }
        __syncthreads();
    };
    for (int t = ts; t < nt; t += 2) {
        tile_body(t, s_k1, s_v0, s_k0, s_v1, s_ksc[1], s_vsc[0], s_ksc[0], s_vsc[1], sa, ka, sb,
                  kb4);
        if (t + 1 < nt)
            tile_body(t + 1, s_k0, s_v1, s_k1, s_v0, s_ksc[0], s_vsc[1], s_ksc[1], s_vsc[0], sb,
                      kb4, sa, ka);
    }

    if (bad)
        s_bad = 1;
    __syncthreads();
    const bool nan = s_bad != 0;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const float inv = PV8 ? __builtin_ldexpf(1.f / row_sum4(l[rt]), vexp)
                              : 1.f / row_sum4(l[rt]);
        if (row[rt] >= n_rows)
            continue;
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

template <int D, bool FP8, int RT, int NW, bool QF8 = false, bool PV8 = false>
hipError_t launch_t(const PrefillArgs& a, hipStream_t stream)
{
    using G = PGeo<D, FP8, RT, NW>;
    const int g = a.n_head / a.n_head_kv;
    const int BP = G::ROWS / g;
    const int npbm = ((a.cu_seqlens ? a.max_q_len : a.n_rows) + BP - 1) / BP;
    const int64_t nblk = (int64_t)(a.cu_seqlens ? a.n_var : 1) * npbm * a.n_head_kv;
    if (nblk > (int64_t)1 << 30)
        return hipErrorInvalidValue;
    const int grid = (int)((nblk + 7) / 8) * 8;
    if (a.ev_start)
        (void)hipEventRecord(a.ev_start, stream);
    hipLaunchKernelGGL((prefill_kernel<D, FP8, RT, NW, QF8, PV8>), dim3(grid), dim3(G::NTH), 0, stream,
                       a);
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
    // One 16-row tile per wave, eight waves: two waves per SIMD, so one
    // wave's softmax overlaps the other's matrix work.  (Two row tiles per
    // wave halve the LDS reads per flop but need more than the 256 VGPRs of
    // a wave at this occupancy for head_dim 256.)
    if (a.qk_fp8 || a.pv_fp8) {
        if (!a.fp8)
            return hipErrorNotSupported;
        const int sel = (a.qk_fp8 ? 1 : 0) | (a.pv_fp8 ? 2 : 0);
        if (sel == 3 && !a.narrow) {
            // Both bits: the two-role kernel where it serves the shape.
            const hipError_t e = launch_prefill_pipe(a, stream);
            if (e != hipErrorNotSupported)
                return e;
        }
        if (a.head_dim == 128) {
            switch (sel) {
            case 1: return launch_t<128, true, 1, 8, true, false>(a, stream);
            case 2: return launch_t<128, true, 1, 8, false, true>(a, stream);
            default: return launch_t<128, true, 1, 8, true, true>(a, stream);
            }
        }
        if (a.head_dim == 256) {
            switch (sel) {
            case 1: return launch_t<256, true, 1, 8, true, false>(a, stream);
            case 2: return launch_t<256, true, 1, 8, false, true>(a, stream);
            default: return launch_t<256, true, 1, 8, true, true>(a, stream);
            }
        }
        return hipErrorNotSupported;
    }
    if (a.narrow && a.fp8 && a.head_dim == 128)
        return launch_t<128, true, 1, 4>(a, stream);
    if (!a.fp8) {
        const hipError_t e = launch_prefill_pipe(a, stream);
        if (e != hipErrorNotSupported)
            return e;
    }
    if (a.head_dim == 128)
        return a.fp8 ? launch_t<128, true, 1, 8>(a, stream) : launch_t<128, false, 1, 8>(a, stream);
    if (a.head_dim == 256)
        return a.fp8 ? launch_t<256, true, 1, 8>(a, stream) : launch_t<256, false, 1, 8>(a, stream);
    return hipErrorNotSupported;
}

}  // namespace pa
