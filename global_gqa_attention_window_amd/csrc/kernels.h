// Launchers of the gfx950 kernels, called by the C ABI (api.hip) after it has
// checked every argument.  Shapes reaching these functions are valid.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/gqa_attn.h"
#include "prologue.h"

size_t decode_workspace_bytes(int S, int Hq, int D, int cap);
// bytes of partials a one-row decode launch (launch_decode) writes and reads:
// one fp32 (max, sum, accumulator[D]) per (stream, query head, run of chunks)
size_t decode_partials_bytes(int S, int Hq, int D, int cap);

// attn_decode's argument checks other than its workspace (api.hip); ATTN_OK
// with S == 0 means there is nothing to launch
int decode_args_status(const void* out, const void* q, const void* k_cache,
                       const void* v_cache, const int32_t* pos, int n_seq, int n_q_heads,
                       int n_kv_heads, int head_dim, int cache_cap, int ring, int window,
                       float scale);

hipError_t launch_decode(uint16_t* out, const uint16_t* q, const uint16_t* kc,
                         const uint16_t* vc, const int32_t* pos, int S, int Hq,
                         int Hkv, int D, int cap, int ring, int window,
                         float scale, void* ws, hipStream_t stream);

// R rows per stream at positions pos[s] .. pos[s] + R - 1 (1 <= R <= 16);
// q, out [S][R][Hq][D]; ws as decode_workspace_bytes(S * R, Hq, D, cap)
// fused: one launch where the merge fits a workgroup; ws then starts with
// ATTN_DECODE_COUNTER_BYTES of counters (zero on entry, left zero)
// prep (one row per stream, else NULL): queries from the stacked rows,
// normed and rotated in place; the row's key and value written first
hipError_t launch_decode_rows(uint16_t* out, const uint16_t* q, const uint16_t* kc,
                              const uint16_t* vc, const int32_t* pos, int S, int R, int Hq,
                              int Hkv, int D, int cap, int ring, int window, float scale,
                              void* ws, bool fused, const PrepArgs* prep, hipStream_t stream);
hipError_t launch_qkv_prep(uint16_t* q_out, const PrepArgs& pa, const int32_t* pos, int S,
                           int Hq, int Hkv, int D, int cap, int ring, hipStream_t stream);
hipError_t launch_decode_counters_init(void* ws, hipStream_t stream);

int prefill_key_block(int D, int p_mode);

// split prompt attention (head dim 256): at most PREFILL_MAX_SPLIT
// workgroups share a tile's key blocks; the count a launch uses, and the
// bytes of partials it writes (one fp32 (max, sum, accumulator[D]) per
// (row, query head, range))
constexpr int PREFILL_MAX_SPLIT = 4;
int prefill_split_count(int n_rows, int Hq, int Hkv, int D);
size_t prefill_partials_bytes(int n_rows, int Hq, int D, int S);

// ws: NULL for one workgroup a tile; else room for
// prefill_partials_bytes(n_rows, Hq, D, PREFILL_MAX_SPLIT), and the launch
// splits a tile's key blocks when few workgroups would fill the chip
hipError_t launch_prefill(uint16_t* out, const uint16_t* q, const uint16_t* kc,
                          const uint16_t* vc, int pos0, int n_rows, int Hq,
                          int Hkv, int D, int cap, int ring, int window,
                          float scale, int p_mode, const int32_t* last_key,
                          void* ws, hipStream_t stream);

// A prompt of n_rows rows in chunks of `chunk`, with the bits of
// launch_cache_write + launch_prefill (no workspace) per chunk, in one
// attention launch: a linear cache takes every row first; a ring's attended
// keys go to a linear copy in ws (prefill_prompt_stage_bytes), and the
// prompt's last rows enter the ring after the attention.
size_t prefill_prompt_stage_bytes(int pos0, int n_rows, int Hkv, int D, int ring, int window);
hipError_t launch_prefill_prompt(uint16_t* out, const uint16_t* q, const uint16_t* k,
                                 const uint16_t* v, uint16_t* kc, uint16_t* vc, int pos0,
                                 int n_rows, int chunk, int Hq, int Hkv, int D, int cap,
                                 int ring, int window, float scale, int p_mode,
                                 const int32_t* last_key, void* ws, hipStream_t stream);

// head dim 512 (prefill512.hip)
hipError_t launch_prefill_512(uint16_t* out, const uint16_t* q, const uint16_t* kc,
                              const uint16_t* vc, int pos0, int n_rows, int Hq, int Hkv,
                              int cap, int ring, int window, float scale, int p_mode,
                              const int32_t* last_key, int base, int clamp_rows,
                              hipStream_t stream);

hipError_t launch_cache_write(uint16_t* kc, uint16_t* vc, const uint16_t* k,
                              const uint16_t* v, int pos0, int n_rows, int Hkv,
                              int D, int cap, int ring, hipStream_t stream);
