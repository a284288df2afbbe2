// kernels.h -- launchers shared between the C-ABI layer (api.cpp) and the
// HIP kernel sources.  Internal; not installed.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

// Tokens per split of the split-K decode/verify kernel: a property of the
// (head_dim, KV dtype) instantiation, 1024 for the fp8 cache at head_dim 128
// (half the split partials to store and combine) and 512 otherwise.  Split
// boundaries sit at absolute multiples of it, so a row's partial results
// depend only on its own position and context -- never on batch size or row
// count.  kChunk, the smallest, sizes workspaces.
constexpr int kChunk = 512;
inline int decode_chunk(int32_t head_dim, bool fp8) { return head_dim == 128 && fp8 ? 1024 : 512; }
// Largest batch the decode/verify kernels take (the per-block prefix over
// sequences lives in LDS).
constexpr int kMaxSeq = 4096;

// The device scratch array of the no-allocation decode entry point
// (scratch.hip): its size, the GPUs it is tracked on, and its address on the
// current GPU (taken once per device with hipGetSymbolAddress).
constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;
hipError_t scratch_address(void** out);

inline int64_t max_splits(int32_t max_pages_per_seq, int32_t page_size)
{
    return ((int64_t)max_pages_per_seq * page_size + kChunk - 1) / kChunk;
}

struct SplitArgs {
    const void* q;
    const void* k_pool;
    const void* v_pool;
    const float* k_scale;
    const float* v_scale;
    int64_t n_pages;
    const int32_t* block_table;
    int32_t max_pages;
    const int32_t* ctx_lens;
    int32_t n_seq, n_head, n_head_kv, head_dim, rows;
    int fp8;
    void* out;
    // Split partials, row-major per (sequence, row): the records of a call
    // with (n_seq, rows) and of one with (n_seq * rows, 1) coincide.
    float* o_part;   // [n_seq][rows][max_split][n_head][head_dim]
    float* ml_part;  // [n_seq][rows][max_split][n_head][2]
    int32_t max_split;
    hipEvent_t ev_start, ev_stop;  // optional timing pair around the split kernel
    int32_t max_blocks;            // grid bound for the split kernel; 0 = fill the device
    // Lower bound on the keys a row attends: row at position p reads keys
    // max(kv_floor[s], p - window + 1) .. p (window 0: no window; kv_floor
    // null: floor 0).  A floor outside 0 .. C - rows gives NaN rows.
    int32_t window;
    const int32_t* kv_floor;
    int32_t slices;  // work items per (sequence, split, kv head); set by the launcher
    // Only the full splits below the one holding the call's first row
    // (0 .. (C - rows) / 512 - 1): the context shared by every row of a round.
    int below_round = 0;
    // 0: split kernel then combine; 1: split kernel only; 2: combine only.
    int phase = 0;
    int32_t chunk_log2;  // log2 of the instantiation's split size; set by the launcher
};

// Decode (rows = 1) and verify (rows = 8): split kernel + fixed-order combine.
hipError_t launch_split_decode(const SplitArgs& a, hipStream_t stream);

struct AppendArgs {
    const void* k_new;
    const void* v_new;
    const int32_t* slots;
    int32_t n_tok;
    void* k_pool;
    void* v_pool;
    float* k_scale;
    float* v_scale;
    int64_t n_pages;
    int32_t n_head_kv, head_dim;
    int fp8;
};
hipError_t launch_append(const AppendArgs& a, hipStream_t stream);

struct PrefillArgs {
    const void* q;
    int32_t n_rows;
    const void* k_pool;
    const void* v_pool;
    const float* k_scale;
    const float* v_scale;
    int64_t n_pages;
    const int32_t* block_table;
    int32_t max_pages;
    int32_t ctx_len;
    int32_t n_head, n_head_kv, head_dim;
    int fp8;
    void* out;
    hipEvent_t ev_start, ev_stop;
    // Several sequences in one launch (the chunk half of a mixed step).  When
    // cu_seqlens is set, sequence i of the launch owns token rows
    // cu_seqlens[i] .. cu_seqlens[i + 1] - 1 of q and out, has ctx_lens[i]
    // keys and block-table row i; n_rows and ctx_len are then unused.  A
    // sequence whose entries are out of range (rows outside 1 .. max_q_len or
    // past n_tok, ctx_len below its rows or past the table) is skipped.
    const int32_t* cu_seqlens;  // device, n_var + 1 entries, or null
    const int32_t* ctx_lens;    // device, n_var entries
    int32_t n_var;              // sequences of the launch
    int32_t max_q_len;          // bound on any sequence's rows (sizes the grid)
    int32_t n_tok;              // token rows of q and out
    // Lower bound on the keys a row attends (one-sequence launch only): row
    // at position p reads keys max(kv_floor, p - window + 1) .. p; window 0
    // means no window.  0 <= kv_floor <= the first row's position.
    int32_t window;
    int32_t kv_floor;
    // fp8 cache only: QK^T on the fp8 matrix unit, K with its stored codes,
    // each query vector rounded to E4M3 at a power-of-two scale.
    int qk_fp8 = 0;
    // fp8 cache only: PV on the fp8 matrix unit, V with its stored codes, P
    // rounded to E4M3 with the tile's V page scales folded in.
    int pv_fp8 = 0;
    // fp8 cache at head_dim 128: workgroups of four waves (64 query rows),
    // which leave a CU room for a decode workgroup beside them.  A row's
    // arithmetic is the same as with eight.
    int narrow = 0;
};
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
// The bf16-cache prefill with score and output waves (prefill_pipe.hip);
// hipErrorNotSupported for the shapes it does not take.
hipError_t launch_prefill_pipe(const PrefillArgs& a, hipStream_t stream);

struct CheckArgs {
    const int32_t* block_table;
    const int32_t* ctx_lens;
    const int32_t* kv_floor;  // or null
    int32_t window;           // 0: none
    int32_t n_seq, rows, max_pages, page_size;
    int64_t n_pages;
    int64_t* err;  // -1, or s * (max_pages + 1) + entry + 1 (entry -1: the length)
};
hipError_t launch_check(const CheckArgs& a, hipStream_t stream);

// Tree-shaped speculative round: per (sequence, row) branch views (tree.hip).
struct TreeArgs {
    const int32_t* block_table;
    const int32_t* ctx_lens;
    const int32_t* tree_mask;  // [n_seq][rows]: bit j = the row attends round row j
    const int32_t* scratch;    // [n_seq][rows][2] pool pages reserved for the views
    void* k_pool;
    void* v_pool;
    float* k_scale;
    float* v_scale;
    int64_t n_pages;
    int32_t n_seq, rows, max_pages, n_head_kv, head_dim;
    int fp8;
    int32_t* vtable;  // out: [n_seq * rows][max_pages]
    int32_t* vlens;   // out: [n_seq * rows]
    int32_t* vfloor;  // out: [n_seq * rows], first key of the split holding C - rows
    int32_t chunk;    // split size of the decode kernels that read the views
};
hipError_t launch_tree_stage(const TreeArgs& a, hipStream_t stream);

}  // namespace pa
