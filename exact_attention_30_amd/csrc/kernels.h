// Launch arguments shared by the kernel files and the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

struct PrefillArgs {
  const uint16_t *q;
  const uint16_t *k;
  const uint16_t *v;
  uint16_t *out;
  float *lse;
  int B, Hq, Hkv, Lq, Lk;
  int G;       // Hq / Hkv
  int hpw;     // query heads per workgroup (divides G and the wave count)
  int wph;     // waves per head = waves / hpw
  int Bq;      // query rows per head per workgroup = rows per wave * wph
  int n_qblk;  // ceil(Lq / Bq)
  int n_hg;    // head groups per KV head = G / hpw
  int total;   // workgroups in the grid (including the key splits)
  int causal;
  float c;     // scale * log2(e)
  int window;       // causal sliding window: a row sees its `window` most recent keys (0: all)
  int nsplit;       // key ranges per query block (1: the kernel writes out and lse itself)
  float *part_o;    // nsplit > 1: [rows][nsplit][D] normalised partial outputs, rows = B * Hq * Lq
  float *part_lse;  // nsplit > 1: [rows][nsplit] partial log-sum-exps (-inf for an empty range)
  int persist;      // > 0: the grid is this many resident workgroups, each taking several work items
};

struct DecodeArgs {
  const uint16_t *q;
  const uint16_t *kc;
  const uint16_t *vc;
  const int32_t *lens;
  uint16_t *out;
  float *lse;
  // int8 caches (kc / vc then hold int8 codes): fp16 scale per 32-element
  // block of each row, [B][Hkv][Lmax][D / 32]; null for bf16 caches
  const uint16_t *kscale;
  const uint16_t *vscale;
  long long *pre;   // [B + 1] prefix sums of 32-key blocks per sequence (planner output)
  float *part_o;    // [slots][GW][D] normalised piece outputs, slots = waves + B * Hkv * n_hg
  float *part_lse;  // [slots][GW] piece log-sum-exps
  int B, Hq, Hkv, Lmax;
  int G;            // Hq / Hkv
  int T;            // query rows per sequence and head (1: plain decode)
  int window;       // sliding window: row t sees its `window` most recent keys (0: all)
  int n_hg;         // groups of up to decode_group(D) query rows per KV head
                    // (a KV head's G * T rows; GW = min(G * T, decode_group(D)))
  float c;          // scale * log2(e)
  int wide;         // 1: decode_wide_kernel (see decode_use_wide)
};

struct BackwardArgs {
  const uint16_t *q;      // [B][Hq][Lq][D]
  const uint16_t *k;      // [B][Hkv][Lk][D]
  const uint16_t *v;
  const uint16_t *out;    // forward output [B][Hq][Lq][D]
  const uint16_t *dout;   // gradient of the loss w.r.t. out
  const float *lse;       // forward log-sum-exp [B][Hq][Lq] (natural log)
  uint16_t *dq;           // [B][Hq][Lq][D]
  uint16_t *dk;           // [B][Hkv][Lk][D]
  uint16_t *dv;
  float *delta;           // workspace [B][Hq][Lq]: <dout_i, out_i>
  float *lse2;            // workspace [B][Hq][Lq]: lse * log2(e)
  int B, Hq, Hkv, Lq, Lk;
  int G;
  int causal;
  int window;
  int dq_hpw;             // query heads per dq workgroup (divides G and 4)
  float scale;
  float c;                // scale * log2(e)
};

// Upper bound on the waves of the decode main kernel (sizes the workspace).
constexpr int kDecodeMaxWaves = 4096;
// Query heads of one KV head handled together by a decode wave (16 per MFMA
// column block); larger groups are split into groups of this size, each read
// of K/V then serving one group.
#ifndef ATTN_DEC_GROUP
#define ATTN_DEC_GROUP 64
#endif
constexpr int kDecodeGroup = ATTN_DEC_GROUP;
// Query rows of one KV head served by one wave at head dim D: kDecodeGroup up
// to D = 128; 32 at D = 256, where the accumulators of more rows do not fit
// beside a block of K and V in a wave's registers.
constexpr int decode_group(int D) { return D == 256 && kDecodeGroup > 32 ? 32 : kDecodeGroup; }

// Fill in the query-row packing (hpw, wph, Bq, n_qblk, n_hg, total) for the
// kernel that serves head dim D, for a.nsplit key ranges per query block;
// false if the grid would be too large.
bool prefill_plan(PrefillArgs &a, int D);
// Keys per tile of the prefill kernel for head dim D.
int prefill_tile_keys(int D);
// Resident workgroups per CU of the prefill kernel for head dim D.
hipError_t prefill_wgs_per_cu(int D, int *out);
// whether the prefill kernel used for head dim D takes several work items per
// workgroup (PrefillArgs::persist)
bool prefill_can_persist(int D);
// Largest key-split count the combine step supports.
constexpr int kPrefillMaxSplits = 64;
hipError_t launch_prefill(const PrefillArgs &a, int D, hipStream_t s);
hipError_t launch_decode(const DecodeArgs &a, int D, int waves, hipStream_t s);
hipError_t decode_waves_per_cu(int D, int GW, bool q8, bool wide, int *out);
// Whether a decode takes decode_wide_kernel: bf16 caches, more than 32 query
// rows per row group (two 32-row blocks per wave), a head dim it is built for,
// and at least kDecodeWideMinBlocks 32-key blocks to split (BLOCKS: an upper
// bound from the shapes), so that every wave gets enough of them to keep its
// two blocks of loads in flight.
constexpr long long kDecodeWideMinBlocks = 32768;
bool decode_use_wide(int D, int GW, bool q8, long long blocks);
hipError_t launch_backward(const BackwardArgs &a, int D, hipStream_t s);
// Query heads handled together by one workgroup of the dq kernel.
int backward_dq_heads(int G);

}  // namespace attn
