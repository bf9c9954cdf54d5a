// Internal declarations shared by the launchers and the kernels of libpagedkv.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

constexpr int kTile = 16;  // tokens per tile (a block holds block_size / 16 tiles; a block of 8
                           // tokens is one 8-token tile, and decode reads two per tile)
constexpr int kWave = 64;  // CDNA wavefront width

// Everything pass 1 and pass 2 of decode need; passed by value to both kernels.
struct DecodeArgs {
    const void* q;              // [S, Hq, D]
    void* out;                  // [S, Hq, D]
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_tables;  // [S, max_blocks]
    const int32_t* context_lens;  // [S]
    float* pieces;              // [units][2][piece_floats]
    int32_t* unit_rec;          // [units][kRecInts]
    int32_t* split_count_end;   // arrivals per split sequence (merge folded in): the
                                // count of the split ending in unit u is split_count_end[-1 - u]
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t group;              // Hq / Hkv
    int32_t rows;               // work rows: Hkv (group kernel) or Hq (per-head kernel)
    int32_t heads_per_row;      // G (group kernel) or 1 (per-head kernel)
    int32_t max_blocks;
    int32_t tiles_per_block;
    int32_t num_blocks;
    int32_t num_units;
    int32_t aligned;            // 1: every row cut into num_units / rows identical ranges
    int32_t waves_per_group;    // rows of one range per workgroup (aligned split only)
    int32_t fused;              // 1: pass 1 merges split sequences itself (no pass 2)
    int32_t keep_cached;        // 1: K/V tiles read with ordinary loads (kept in L2 / MALL)
    float scale_log2e;          // scale * log2(e): scores are kept in base-2 units
    // Decode step (pa_decode_step): the step's writes are folded into the launch.
    // Workgroup 0 first copies lens_in into context_lens, sets each sequence's table
    // entry for the block of its new token and fills seq_info; every workgroup waits
    // for that (sync[0]) before reading any of them.  Waves reading a tile of a
    // sequence's last block take its new token from k_new / v_new and write it (and
    // a copy-on-write copy) to the cache.
    const int32_t* lens_in;     // [S] context lengths including the step's token (host or device)
    const int64_t* new_slots;   // [S] slot of sequence i's new token (position lens_in[i] - 1), -1 = none
    const int32_t* cow_in;      // [S][2] (src, dst) copy-on-write pair of sequence i, or NULL
    const void* k_new;          // [S, Hkv, D] the step's new keys and values
    const void* v_new;
    int32_t* lens_dev;          // context_lens, written by workgroup 0
    int32_t* tables_dev;        // block_tables, written by workgroup 0
    int32_t* seq_info;          // [S][4]: read block, write block of the last block; flags
    int32_t* sync;              // [4]: released flag, workgroups past it, spin time-outs
    int32_t block_size;
};

// Everything the chunked-prefill kernel needs; passed by value.
struct PrefillArgs {
    const void* q;                // [T, Hq, D]
    void* out;                    // [T, Hq, D]
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_tables;  // [S, max_blocks]
    const int32_t* query_start;   // [S + 1]
    const int32_t* context_lens;  // [S]
    int32_t num_seqs;
    int32_t num_tokens;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t max_blocks;
    int32_t tiles_per_block;
    int32_t num_blocks;
    int32_t qgroups;              // workgroups per (sequence, KV head)
    int32_t num_groups;           // num_seqs * num_kv_heads * qgroups
    float scale_log2e;
    int32_t block_size;
};

constexpr int kRecInts = 8;  // per-unit record: row, seq, first unit, last unit of the split ending there
// Decode step: polls of the metadata flag before a workgroup gives up waiting (each
// poll sleeps ~128 clocks, so about 0.1 s): only a launch whose workgroup 0 never
// ran could reach it.
constexpr int kStepSpinLimit = 1 << 20;
// Aligned split: a sequence with n tiles costs kTileCost n + kPieceCost.  Measured on
// the batch-256 GQA workload, a unit's time grows by about 0.8 of a tile per extra
// sequence (piece) in its range, so a piece is charged one tile.
constexpr int kTileCost = 4;
constexpr int kPieceCost = 4;
// Per-head decode with streamed loads: the rows of a workgroup meet at every tile when
// the batch averages at least this many 16-token tiles per sequence (long walks);
// otherwise they run free.  With cached loads they always meet.
constexpr int kBarrierTilesPerSeq = 64;

// Floats of one partial-result record: heads_per_row * (D accumulators + max + sum).
inline size_t piece_floats(int heads_per_row, int head_dim) {
    return static_cast<size_t>(heads_per_row) * (head_dim + 2);
}

hipError_t launch_reshape_and_cache(int dtype, int head_dim, int block_size, int num_kv_heads,
                                    int num_blocks, const void* k, const void* v,
                                    const int64_t* slots, int num_tokens, void* k_cache,
                                    void* v_cache, hipStream_t stream);
hipError_t launch_append_tokens(int dtype, int head_dim, int block_size, int num_kv_heads,
                                int num_blocks, const void* k, const void* v,
                                const int64_t* slots, const int32_t* cow, int num_tokens,
                                void* k_cache, void* v_cache, int32_t* tables, int rows, int cols,
                                const int32_t* upd, int num_updates, const int32_t* lens_in,
                                int32_t* lens_out, int num_lens, hipStream_t stream);
hipError_t launch_copy_blocks(int dtype, int head_dim, int block_size, int num_kv_heads,
                              int num_blocks, void* k_cache, void* v_cache, const int32_t* pairs,
                              int num_pairs, hipStream_t stream);
hipError_t launch_swap_blocks(int dtype, int head_dim, int block_size, int num_kv_heads,
                              const void* src_k, const void* src_v, int src_blocks, void* dst_k,
                              void* dst_v, int dst_blocks, const int32_t* pairs, int num_pairs,
                              hipStream_t stream);
hipError_t launch_update_block_tables(int32_t* tables, int rows, int cols, const int32_t* upd,
                                      int n, hipStream_t stream);
// passes: bit 0 = pass 1 (tiles -> outputs / partial records), bit 1 = pass 2 (merge).
// Returns hipErrorInvalidValue for an uncompiled (dtype, head_dim, group) combination.
// Chunked-prefill attention (bf16, D in {64, 128}, G in {1, 2, 4, 8, 16}).
hipError_t launch_prefill(int head_dim, int group, int max_query_len, PrefillArgs& a,
                          hipStream_t stream);
hipError_t launch_decode(int dtype, int head_dim, bool use_group_kernel, const DecodeArgs& a,
                         int passes, hipStream_t stream);
// One decode step with its cache writes folded in (the single-kernel decode with
// DecodeArgs' step fields set).
hipError_t launch_decode_step(int dtype, int head_dim, bool use_group_kernel, const DecodeArgs& a,
                              hipStream_t stream);
// The decode kernels of one variant: Stream = non-temporal K/V loads, Step = the
// decode step, Half = blocks of 8 tokens (instantiated in decode_variant.hip).
template <bool Stream, bool Step, bool Half>
hipError_t launch_decode_variant(int dtype, int head_dim, bool use_group_kernel, const DecodeArgs& a,
                                 int passes, hipStream_t stream);

}  // namespace pkv
