// Backward: dq, dk, dv of exact GQA attention from the forward's out and lse.
//
// Method (pages, by title): "어텐션 구현 고르기, SDPA·FlashAttention 메모리와
// GPU 비용", section "eager 어텐션 메모리, 길이에 따라 얼마나 커지나" (training
// keeps a score table per layer for the backward pass; FlashAttention keeps
// only per-row statistics instead); the gradients are the chain rule through
// the forward definition: with p_ij = exp(scale s_ij - lse_i),
//   dv_j = sum_i p_ij dout_i,  dp_ij = <dout_i, v_j>,
//   ds_ij = p_ij (dp_ij - delta_i),  delta_i = <dout_i, out_i>,
//   dq_i = scale sum_j ds_ij k_j,  dk_j = scale sum_i ds_ij q_i,
// summed over the G query heads of a KV head for dk and dv.
//
// gfx950 design
//  * No score table: every tile of p is recomputed from q, k and the saved
//    lse (one exp2 per element), as the forward never stored it.
//  * dk/dv kernel for D = 64 and 128 (bwd_dkdv2_kernel): pairs of waves on one
//    SIMD own 32 keys; one wave of a pair forms S, P (handed to its partner
//    through LDS) and dV, the other dP, dS and dK, so each holds one operand
//    and one accumulator set and two waves fit per SIMD.
//  * dk/dv kernel for D = 256 (bwd_dkdv_kernel): a wave owns 32 keys of one KV head and keeps their k and v
//    rows as MFMA operands in registers; the workgroup (4 waves, 128 keys)
//    walks 64-row stages of all G query heads that read the KV head, moving
//    q, dout, lse and delta straight from global memory into LDS (direct
//    loads, three stages in flight).  Per 32-row half and wave, four
//    v_mfma_f32_32x32x16_bf16 chains: S = Q K^T and dP = dO V^T (queries on
//    M, keys on N), then dV^T += dO^T P and dK^T += Q^T dS, where P and dS
//    come straight from the S / dP accumulators (a lane holds one key column)
//    and dO^T, Q^T are read with ds_read_b64_tr_b16.  The two halves of an
//    unmasked stage are software-pipelined.  dk and dv of a KV head are
//    complete in one workgroup: no atomics.
//  * dq kernels: a wave owns 32 query rows (q and dout rows as operands in
//    registers) and walks the 32-key tiles in reach of its rows: S^T = K Q^T,
//    dP^T = V dO^T, then dQ^T += K^T dS^T with K^T read transposed from the
//    same LDS tile.  For D = 64 and 128 (bwd_dq2_kernel) eight waves form two
//    groups whose matrix and vector work alternate on each SIMD; for D = 256
//    (bwd_dq_kernel) four waves, one per SIMD.
//  * LDS operand reads are issued several MFMAs ahead of their use.
//  * A tile that is read both row-wise (b128) and transposed (tr16) is stored
//    with a 16-byte-chunk XOR swizzle that keeps both access patterns free of
//    bank conflicts (tswz).
//  * Causal (bottom-right) and window masks: query or key tiles that no row
//    or key of a wave can see are skipped; the mask is applied per element
//    only on tiles that cross a boundary.
#include <mutex>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace attn {
namespace {

// XOR on the 16-byte chunk index of row r of a tile read both by rows
// (b128: 16 consecutive rows, one chunk each) and transposed (tr16: 4
// consecutive rows, 64 bytes each): D = 64 rows are 128 bytes long, larger
// rows a multiple of 256 bytes.
template <int D>
ATTN_DEV int tswz(int r) {
  return D == 64 ? 4 * ((r >> 1) & 1) + ((r >> 2) & 3) : 4 * (r & 3) + ((r >> 2) & 3);
}

// element offset of logical chunk c (8 bf16) of row r in a swizzled tile
template <int D>
ATTN_DEV int toff(int r, int c) {
  return r * D + 8 * (c ^ tswz<D>(r));
}

ATTN_DEV bf16x8 tr_operand(const uint16_t *lo, const uint16_t *hi) {
  const bf16x4 a = lds_tr16(lo);
  const bf16x4 b = lds_tr16(hi);
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Scheduling of a run of N MFMAs that each take R operands read from LDS:
// the first AHEAD MFMAs' reads go first, then every MFMA is followed by the
// reads of the MFMA AHEAD places later, so that LDS latency hides behind
// matrix work (AHEAD = 0: left to the compiler).
template <int N, int R, int AHEAD>
ATTN_DEV void sched_reads_ahead() {
  if constexpr (AHEAD > 0) {
    __builtin_amdgcn_sched_group_barrier(0x100, R * AHEAD, 0);
#pragma unroll
    for (int i = 0; i < N - AHEAD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
  }
}

// The same, with V VALU instructions placed after every MFMA of the run
// (work of another stage that does not feed these MFMAs).
template <int N, int R, int AHEAD, int V>
ATTN_DEV void sched_interleave() {
  __builtin_amdgcn_sched_group_barrier(0x100, R * AHEAD, 0);
#pragma unroll
  for (int i = 0; i < N - AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
  }
#pragma unroll
  for (int i = 0; i < AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
  }
}

}  // namespace

//  ATTN_BWD_PAIRS      dk/dv for D = 64 and 128 on bwd_dkdv2_kernel (paired waves)
#ifndef ATTN_BWD_PAIRS
#define ATTN_BWD_PAIRS 1
#endif
//  ATTN_BWD_PIPE       dk/dv: both halves of an unmasked stage software-pipelined
//  ATTN_BWD_VALU_PER   VALU instructions scheduled after each MFMA there
#ifndef ATTN_BWD_PIPE
#define ATTN_BWD_PIPE 1
#endif
#ifndef ATTN_BWD_VALU_PER
#define ATTN_BWD_VALU_PER 6
#endif
//  ATTN_BWD_PAIR_LOADS paired dk/dv, which waves stage the query tiles: 0 every wave at
//                      the start of a stage; 1 the dP/dS waves there (the S/P waves
//                      hold the first phase's critical path); 2 the S/P waves in their
//                      second phase, between the dV products of the two halves (where
//                      they wait for their partners anyway)
#ifndef ATTN_BWD_PAIR_LOADS
#define ATTN_BWD_PAIR_LOADS 2
#endif
//  ATTN_BWD_DQ_PAIRS   dq for D = 64 and 128 on bwd_dq2_kernel (two groups of waves)
#ifndef ATTN_BWD_DQ_PAIRS
#define ATTN_BWD_DQ_PAIRS 1
#endif
//  ATTN_BWD_P_PIPE64 / ATTN_BWD_P_PIPE128   paired dk/dv at D = 64 / 128: the S/P wave
//                      exponentiates the first half beside the second half's S products
//                      (unmasked stages), this many vector instructions after each MFMA
//                      (0: halves one after the other)
#ifndef ATTN_BWD_P_PIPE64
#define ATTN_BWD_P_PIPE64 2
#endif
#ifndef ATTN_BWD_P_PIPE128
#define ATTN_BWD_P_PIPE128 6
#endif
//  ATTN_BWD_QK_AHEAD   operand reads of the S / dP products issued this many MFMAs ahead
//  ATTN_BWD_TR_AHEAD   transposed operand reads of the dV / dK / dQ products, likewise
#ifndef ATTN_BWD_QK_AHEAD
#define ATTN_BWD_QK_AHEAD 6
#endif
#ifndef ATTN_BWD_TR_AHEAD
#define ATTN_BWD_TR_AHEAD 4
#endif
//  ATTN_BWD_XPIPE256   bwd_dkdv_kernel at D = 256: the S and dP MFMAs take their
//                      operand reads ATTN_BWD_XAHEAD MFMAs ahead, in explicit
//                      program order held by scheduling fences (the scheduler had
//                      put every read right before its MFMA); the same for the
//                      dV/dK products spills 16 registers, so those stay as they are
#ifndef ATTN_BWD_XPIPE256
#define ATTN_BWD_XPIPE256 1
#endif
#ifndef ATTN_BWD_XAHEAD
#define ATTN_BWD_XAHEAD 2
#endif
template <int D>
constexpr bool kBwdXPipeS = D == 256 && ATTN_BWD_XPIPE256 != 0;
constexpr int kBwdXAhead = ATTN_BWD_XAHEAD;
// D = 256 leaves fewer registers for reads in flight
template <int D>
constexpr int kQkAhead = D == 256 ? 2 : ATTN_BWD_QK_AHEAD;
template <int D>
constexpr int kTrAhead = D == 256 ? 1 : ATTN_BWD_TR_AHEAD;

// ---------------------------------------------------------------------------
// delta_i = <dout_i, out_i> (fp32), and lse_i * log2(e); one wave per row.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BackwardArgs a) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const long long rows = (long long)a.B * a.Hq * a.Lq;
  if (row >= rows) return;
  const uint16_t *o = a.out + row * D;
  const uint16_t *g = a.dout + row * D;
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < D / 64; ++i) {
    const float x = (float)__builtin_bit_cast(__bf16, o[lane + 64 * i]);
    const float y = (float)__builtin_bit_cast(__bf16, g[lane + 64 * i]);
    s = __builtin_fmaf(x, y, s);
  }
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) s += __shfl_xor(s, sh);
  if (lane == 0) {
    a.delta[row] = s;
    a.lse2[row] = a.lse[row] * ATTN_LOG2E;
  }
}

// ---------------------------------------------------------------------------
// dk / dv
// ---------------------------------------------------------------------------
constexpr int kBwdWaves = 4;
constexpr int kBwdKeys = 32 * kBwdWaves;   // keys per dk/dv workgroup
// query rows per stage of the dk/dv loop: two halves of 32 (D = 256: one half,
// so that three stages fit in LDS)
template <int D>
constexpr int kBwdRows = D == 256 ? 32 : 64;


// s_waitcnt vmcnt(n) for n < 16 (expcnt and lgkmcnt left alone)
#define ATTN_BWD_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(0x0F70 | (n))

// One direct global->LDS load of 16 (or 4) bytes per lane: lane i writes
// bytes [size i, size (i + 1)) after the wave-uniform LDS address `lds`.
template <int SIZE>
ATTN_DEV void dma_to_lds(const void *g, void *lds) {
  auto *gp = (__attribute__((address_space(1))) void *)const_cast<void *>(g);
  auto *lp = (__attribute__((address_space(3))) void *)lds;
  if constexpr (SIZE == 16) __builtin_amdgcn_global_load_lds(gp, lp, 16, 0, 0);
  else __builtin_amdgcn_global_load_lds(gp, lp, 4, 0, 0);
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1))) void bwd_dkdv_kernel(BackwardArgs a) {
  constexpr int ROWS = kBwdRows<D>;
  constexpr int TILE = ROWS * D;              // elements of a q (or dout) stage
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  constexpr int RPB = 512 / D;                // rows per 1 KiB direct load
  constexpr int BPW = TILE * 2 / 1024 / kBwdWaves;   // 1 KiB blocks per wave per tensor and stage
  static_assert(BPW * kBwdWaves * 1024 == TILE * 2, "stage must split evenly over the waves");
  // three stages, each its own array (so that reads of one stage never wait
  // for the direct loads still filling another): q, dout, and the rows'
  // lse * log2(e) (floats 0..63) and delta (floats 64..127)
  __shared__ __attribute__((aligned(1024))) uint16_t qa[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t qb[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t qc[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t da[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t db_[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t dc[TILE];
  __shared__ __attribute__((aligned(256))) float sa[2 * ROWS];
  __shared__ __attribute__((aligned(256))) float sb[2 * ROWS];
  __shared__ __attribute__((aligned(256))) float sc_[2 * ROWS];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int ql = lane & 31, hh = lane >> 5, g16 = lane >> 4, j16 = lane & 15;

  // workgroup -> (key block, b, hkv): the key blocks with the most visible
  // query rows (causal: the first ones) of every head start first
  const int nbh = a.B * a.Hkv;
  const int t = blockIdx.x;
  const int kbk = t / nbh;
  const int bh = t - kbk * nbh;                // b * Hkv + hkv
  const int b = bh / a.Hkv, hkv = bh - b * a.Hkv;
  const int j0 = kbk * kBwdKeys;
  const int kw0 = j0 + 32 * w;                 // this wave's first key
  const int key = kw0 + ql;                    // this lane's key (column)
  const int off = a.Lk - a.Lq;
  const int win = a.window;

  // k and v rows of the wave's keys as B operands: lane (ql, hh) holds key
  // kw0 + ql, dims 16 ks + 8 hh ...
  const size_t kvbase = ((size_t)b * a.Hkv + hkv) * (size_t)a.Lk * D;
  bf16x8 kf[D / 16], vf[D / 16];
  {
    const u32x4 z = {0u, 0u, 0u, 0u};
    const bool in = key < a.Lk;
    const uint16_t *kp = a.k + kvbase + (size_t)(in ? key : 0) * D + 8 * hh;
    const uint16_t *vp = a.v + kvbase + (size_t)(in ? key : 0) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      kf[ks] = as_bf16x8(in ? ld16(kp + 16 * ks) : z);
      vf[ks] = as_bf16x8(in ? ld16(vp + 16 * ks) : z);
    }
  }

  // query rows that see some key of this workgroup (the same for every head)
  int qlo = 0, qhi = a.Lq;
  if (a.causal) {
    qlo = max(0, j0 - off);
    if (win) qhi = min(a.Lq, j0 + kBwdKeys - 1 - off + win);
  }
  qlo = qlo / 32 * 32;
  const int ntile_h = qhi > qlo ? (qhi - qlo + ROWS - 1) / ROWS : 0;
  const int ntile = ntile_h * a.G;

  // per-lane LDS offsets: b128 operand (row ql, chunk 2 ks + hh) and the
  // transposed operand (rows 4 hh + (j16 >> 2) [+8], 4 columns at
  // 32 db + 16 (g16 & 1) + 4 (j16 & 3)); a 16-row step adds 16 D.
  // the swizzle touches only the low 4 bits of a chunk index, so from 16
  // chunks on the offsets repeat 128 elements further: 8 (and 4 + 4) of them
  // are kept, the rest is an immediate offset of the read
  constexpr int NRO = D / 16 < 8 ? D / 16 : 8, NTO = D / 32 < 4 ? D / 32 : 4;
  int roff8[NRO];
#pragma unroll
  for (int ks = 0; ks < NRO; ++ks) roff8[ks] = toff<D>(ql, 2 * ks + hh);
  int tlo4[NTO], thi4[NTO];
  {
    const int r = 4 * hh + (j16 >> 2);
    const int c = 2 * (g16 & 1) + ((j16 & 3) >> 1);
#pragma unroll
    for (int dd = 0; dd < NTO; ++dd) {
      tlo4[dd] = toff<D>(r, 4 * dd + c) + 4 * (j16 & 1);
      thi4[dd] = toff<D>(r + 8, 4 * dd + c) + 4 * (j16 & 1);
    }
  }
  auto roff = [&](int ks) __attribute__((always_inline)) { return roff8[ks % NRO] + (ks / NRO) * 128; };
  auto tlo = [&](int dd) __attribute__((always_inline)) { return tlo4[dd % NTO] + (dd / NTO) * 128; };
  auto thi = [&](int dd) __attribute__((always_inline)) { return thi4[dd % NTO] + (dd / NTO) * 128; };

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }

  // Stage tile tt (head, ROWS rows) straight from global memory into LDS: each
  // wave moves BPW blocks of 1 KiB of q and of dout (lane i fills bytes
  // [16 i, 16 i + 16) of a block, so it fetches the logical chunk that the
  // swizzle puts there; rows past the end are read from the last row and
  // masked in compute), and waves 0 and 1 move the rows' lse and delta
  // (one float per lane).  Per tile a wave issues 2 BPW loads (+1 for waves
  // 0 and 1).
  auto issue = [&](int tt, uint16_t *qd, uint16_t *dd, float *sd) __attribute__((always_inline)) {
    const int hq = hkv * a.G + tt / ntile_h;
    const int i0 = qlo + (tt % ntile_h) * ROWS;
    const size_t rowbase = ((size_t)b * a.Hq + hq) * a.Lq;
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int blk = wu * BPW + i;
      const int row = blk * RPB + lane / CPR;
      const int c = (lane % CPR) ^ tswz<D>(row);
      const size_t grow = rowbase + min(i0 + row, a.Lq - 1);
      dma_to_lds<16>(a.q + grow * D + 8 * c, qd + blk * 512);
      dma_to_lds<16>(a.dout + grow * D + 8 * c, dd + blk * 512);
    }
    if (wu < 2) {
      // one float per lane (ROWS lanes)
      const float *src = wu == 0 ? a.lse2 : a.delta;
      const size_t grow = rowbase + min(i0 + lane, a.Lq - 1);
      if (ROWS == 64 || lane < ROWS) dma_to_lds<4>(src + grow, sd + ROWS * wu);
    }
  };
  auto wait_tile = [&](bool younger) __attribute__((always_inline)) {
    if (younger) {
      if (wu < 2) ATTN_BWD_WAIT_VM(2 * BPW + 1);
      else ATTN_BWD_WAIT_VM(2 * BPW);
    } else {
      ATTN_BWD_WAIT_VM(0);
    }
  };

  const float c = a.c;
  // A half (32 rows starting at i0h) of a staged tile: skipped when it lies
  // past the rows or no row of it sees a key of this wave; masked per
  // element when it crosses a mask boundary or the end of the rows.
  auto skip_half = [&](int i0h) __attribute__((always_inline)) {
    if (i0h >= a.Lq) return true;
    return a.causal && (i0h + 31 + off < kw0 || (win && i0h + off - win + 1 > kw0 + 31));
  };
  auto cross_half = [&](int i0h) __attribute__((always_inline)) {
    return i0h + 31 >= a.Lq || (a.causal && (i0h + off < kw0 + 31 || (win && i0h + 31 + off - win + 1 > kw0)));
  };
  // S = Q K^T and dP = dO V^T of one half (qt, dt at the half's first row)
  auto sdp = [&](const uint16_t *qt, const uint16_t *dt, f32x16 &s, f32x16 &dp) __attribute__((always_inline)) {
    s = f32x16{};
    dp = f32x16{};
    if constexpr (kBwdXPipeS<D>) {
      // operand reads A MFMAs ahead in a ring of A + 1, S and dP alternating
      constexpr int N = 2 * (D / 16), A = kBwdXAhead;
      auto rd = [&](int i) __attribute__((always_inline)) { return ld16((i & 1 ? dt : qt) + roff(i >> 1)); };
      u32x4 r[A + 1];
#pragma unroll
      for (int i = 0; i < A; ++i) r[i] = rd(i);
#pragma unroll
      for (int i = 0; i < N; ++i) {
        if (i + A < N) r[(i + A) % (A + 1)] = rd(i + A);
        __builtin_amdgcn_sched_barrier(0);
        if (i & 1) dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(r[i % (A + 1)]), vf[i >> 1], dp, 0, 0, 0);
        else s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(r[i % (A + 1)]), kf[i >> 1], s, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      return;
    }
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ld16(qt + roff(ks))), kf[ks], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ld16(dt + roff(ks))), vf[ks], dp, 0, 0, 0);
    }
  };
  // p and ds of one half as bf16 B operands; this lane: key column `key`,
  // rows i0h + 8 (rr >> 2) + 4 hh + (rr & 3)
  auto soft = [&](const float *st, int rb, int i0h, const f32x16 &s, const f32x16 &dp, bf16x8(&pb)[2],
                  bf16x8(&sb)[2], bool crosses) __attribute__((always_inline)) {
    float pv[16], dsv[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int r = 8 * (rr >> 2) + 4 * hh + (rr & 3);
      float pe = fast_exp2(__builtin_fmaf(s[rr], c, -st[32 * rb + r]));
      if (crosses) {
        const int i = i0h + r;
        const int lim = i + off;
        const bool vis = i < a.Lq && (!a.causal || (key <= lim && (!win || key > lim - win)));
        pe = vis ? pe : 0.f;
      }
      pv[rr] = pe;
      dsv[rr] = pe * (dp[rr] - st[ROWS + 32 * rb + r]);
    }
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
      pb[qh] = pack8(pv[8 * qh], pv[8 * qh + 1], pv[8 * qh + 2], pv[8 * qh + 3], pv[8 * qh + 4], pv[8 * qh + 5],
                     pv[8 * qh + 6], pv[8 * qh + 7]);
      sb[qh] = pack8(dsv[8 * qh], dsv[8 * qh + 1], dsv[8 * qh + 2], dsv[8 * qh + 3], dsv[8 * qh + 4],
                     dsv[8 * qh + 5], dsv[8 * qh + 6], dsv[8 * qh + 7]);
    }
  };
  // dV^T += dO^T P,  dK^T += Q^T dS  (k = the half's query rows)
  auto upd = [&](const uint16_t *qt, const uint16_t *dt, const bf16x8(&pb)[2], const bf16x8(&sb)[2])
      __attribute__((always_inline)) {
#pragma unroll
    for (int dd = 0; dd < D / 32; ++dd) {
#pragma unroll
      for (int qh = 0; qh < 2; ++qh) {
        dv[dd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            tr_operand(dt + 16 * qh * D + tlo(dd), dt + 16 * qh * D + thi(dd)), pb[qh], dv[dd], 0, 0, 0);
        dk[dd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            tr_operand(qt + 16 * qh * D + tlo(dd), qt + 16 * qh * D + thi(dd)), sb[qh], dk[dd], 0, 0, 0);
      }
    }
  };
  // one half on its own
  auto half = [&](const uint16_t *qt, const uint16_t *dt, const float *st, int i0h, int rb) __attribute__((
                                                                                              always_inline)) {
    if (skip_half(i0h)) return;
    qt += rb * 32 * D;
    dt += rb * 32 * D;
    f32x16 s, dp;
    sdp(qt, dt, s, dp);
    sched_reads_ahead<2 * (D / 16), 1, kQkAhead<D>>();
    bf16x8 pb[2], sb2[2];
    soft(st, rb, i0h, s, dp, pb, sb2, cross_half(i0h));
    upd(qt, dt, pb, sb2);
    sched_reads_ahead<4 * (D / 32), 2, kTrAhead<D>>();
  };
  // both halves, neither masked: software-pipelined so that the exponentials
  // of one half run beside the MFMAs of the other
  auto both = [&](const uint16_t *qt, const uint16_t *dt, const float *st, int i0, bool m0, bool m1)
      __attribute__((always_inline)) {
    f32x16 s0, dp0, s1, dp1;
    bf16x8 pb0[2], sb0[2], pb1[2], sb1[2];
    sdp(qt, dt, s0, dp0);
    sched_reads_ahead<2 * (D / 16), 1, kQkAhead<D>>();
    sdp(qt + 32 * D, dt + 32 * D, s1, dp1);
    soft(st, 0, i0, s0, dp0, pb0, sb0, m0);
    sched_interleave<2 * (D / 16), 1, kQkAhead<D>, ATTN_BWD_VALU_PER>();
    upd(qt, dt, pb0, sb0);
    soft(st, 1, i0 + 32, s1, dp1, pb1, sb1, m1);
    sched_interleave<4 * (D / 32), 2, kTrAhead<D>, ATTN_BWD_VALU_PER>();
    upd(qt + 32 * D, dt + 32 * D, pb1, sb1);
    sched_reads_ahead<4 * (D / 32), 2, kTrAhead<D>>();
  };
  auto step = [&](int tt, const uint16_t *qt, const uint16_t *dt, const float *st, uint16_t *qn, uint16_t *dn,
                  float *sn) __attribute__((always_inline)) {
    wait_tile(tt + 1 < ntile);
    barrier_keep_loads();
    if (tt + 2 < ntile) issue(tt + 2, qn, dn, sn);
    const int i0 = qlo + (tt % ntile_h) * ROWS;
    if constexpr (ROWS == 32) {
      half(qt, dt, st, i0, 0);
    } else if (ATTN_BWD_PIPE && !skip_half(i0) && !skip_half(i0 + 32) && !cross_half(i0) && !cross_half(i0 + 32)) {
      both(qt, dt, st, i0, false, false);
    } else {
      half(qt, dt, st, i0, 0);
      half(qt, dt, st, i0 + 32, 1);
    }
  };

  // the k/v operand loads complete before any staged load is issued, so no
  // wait for them is left inside the loop (where it would also drain the
  // stages in flight)
  ATTN_BWD_WAIT_VM(0);
  if (ntile > 0) {
    issue(0, qa, da, sa);
    if (ntile > 1) issue(1, qb, db_, sb);
    for (int tt = 0; tt < ntile; tt += 3) {
      step(tt, qa, da, sa, qc, dc, sc_);
      if (tt + 1 >= ntile) break;
      step(tt + 1, qb, db_, sb, qa, da, sa);
      if (tt + 2 >= ntile) break;
      step(tt + 2, qc, dc, sc_, qb, db_, sb);
    }
  }

  // dk = scale dK, dv = dV; lane: key column, dims 32 dd + 8 j + 4 hh + (0..3)
  if (key < a.Lk) {
    uint16_t *kp = a.dk + kvbase + (size_t)key * D;
    uint16_t *vp = a.dv + kvbase + (size_t)key * D;
    const float scl = a.scale;
#pragma unroll
    for (int dd = 0; dd < D / 32; ++dd)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * dd + 8 * j + 4 * hh;
        bf16x4 kk4, vv4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          kk4[i] = (__bf16)(dk[dd][4 * j + i] * scl);
          vv4[i] = (__bf16)(dv[dd][4 * j + i]);
        }
        *reinterpret_cast<bf16x4 *>(kp + d) = kk4;
        *reinterpret_cast<bf16x4 *>(vp + d) = vv4;
      }
  }
}

// ---------------------------------------------------------------------------
// dk / dv with paired waves (D = 64, 128)
// ---------------------------------------------------------------------------
// Eight waves, two per SIMD: wave w (w < 4) and wave w + 4 share a SIMD and
// own the same 32 keys.  Wave w keeps the keys' k rows, forms S = Q K^T and
// P = exp2(S c - lse2), hands P to its partner through LDS and accumulates
// dV^T += dO^T P; wave w + 4 keeps the v rows, forms dP = dO V^T, then
// dS = P (dP - delta) with the partner's P, and accumulates dK^T += Q^T dS.
// Each wave thus holds one operand set and one accumulator set (about half
// the registers of a wave doing all four products), so two fit per SIMD and
// the exponentials of one run beside the MFMAs of the other.  Per 64-row
// stage: [P-waves: S, P -> LDS | partner: dP], barrier, [P-waves: dV, with
// the direct loads of the stage after next between its two halves |
// partner: dS, dK]; the same products as bwd_dkdv_kernel, in the same order
// per accumulator (bit-identical results).
template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dkdv2_kernel(BackwardArgs a) {
  constexpr int NW = 8;
  constexpr int ROWS = 64;                    // query rows per stage: two halves of 32
  constexpr int TILE = ROWS * D;
  constexpr int CPR = D / 8;
  constexpr int RPB = 512 / D;
  constexpr int BPW = TILE * 2 / 1024 / NW;   // 1 KiB blocks per wave per tensor and stage
  static_assert(BPW * NW * 1024 == TILE * 2, "stage must split evenly over the waves");
  constexpr int NL = ATTN_BWD_PAIR_LOADS ? NW / 2 : NW;   // waves that stage the query tiles
  constexpr int BPL = TILE * 2 / 1024 / NL;              // their 1 KiB blocks per tensor and stage
  __shared__ __attribute__((aligned(1024))) uint16_t qa[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t qb[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t qc[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t da[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t db_[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t dc[TILE];
  __shared__ __attribute__((aligned(256))) float sa[2 * ROWS];
  __shared__ __attribute__((aligned(256))) float sb[2 * ROWS];
  __shared__ __attribute__((aligned(256))) float sc_[2 * ROWS];
  // P of each pair and half: element rr of lane l at [(rr / 4) * 64 + l][rr % 4]
  __shared__ __attribute__((aligned(1024))) float pbuf[4][2][16 * 64];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int pair = wu & 3;
  const bool pwave = wu < 4;                   // forms P and dV (else dP, dS and dK)
  // index among the staging waves (< 0: none)
  const int lw = ATTN_BWD_PAIR_LOADS == 2 ? (pwave ? wu : -1) : wu - (NW - NL);
  const int ql = lane & 31, hh = lane >> 5, g16 = lane >> 4, j16 = lane & 15;

  const int nbh = a.B * a.Hkv;
  const int t = blockIdx.x;
  const int kbk = t / nbh;
  const int bh = t - kbk * nbh;
  const int b = bh / a.Hkv, hkv = bh - b * a.Hkv;
  const int j0 = kbk * kBwdKeys;
  const int kw0 = j0 + 32 * pair;              // the pair's first key
  const int key = kw0 + ql;                    // this lane's key (column)
  const int off = a.Lk - a.Lq;
  const int win = a.window;

  // k rows (P-waves) or v rows (partners) of the pair's keys as B operands
  const size_t kvbase = ((size_t)b * a.Hkv + hkv) * (size_t)a.Lk * D;
  bf16x8 kvf[D / 16];
  {
    const u32x4 z = {0u, 0u, 0u, 0u};
    const bool in = key < a.Lk;
    const uint16_t *src = (pwave ? a.k : a.v) + kvbase + (size_t)(in ? key : 0) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) kvf[ks] = as_bf16x8(in ? ld16(src + 16 * ks) : z);
  }

  int qlo = 0, qhi = a.Lq;
  if (a.causal) {
    qlo = max(0, j0 - off);
    if (win) qhi = min(a.Lq, j0 + kBwdKeys - 1 - off + win);
  }
  qlo = qlo / 32 * 32;
  const int ntile_h = qhi > qlo ? (qhi - qlo + ROWS - 1) / ROWS : 0;
  const int ntile = ntile_h * a.G;

  int roff[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) roff[ks] = toff<D>(ql, 2 * ks + hh);
  int tlo[D / 32], thi[D / 32];
  {
    const int r = 4 * hh + (j16 >> 2);
    const int c = 2 * (g16 & 1) + ((j16 & 3) >> 1);
#pragma unroll
    for (int dd = 0; dd < D / 32; ++dd) {
      tlo[dd] = toff<D>(r, 4 * dd + c) + 4 * (j16 & 1);
      thi[dd] = toff<D>(r + 8, 4 * dd + c) + 4 * (j16 & 1);
    }
  }

  f32x16 acc[D / 32];   // dV^T (P-waves) or dK^T (partners)
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};

  // stage tile tt into LDS (as bwd_dkdv_kernel, the work spread over 8 waves)
  auto issue = [&](int tt, uint16_t *qd, uint16_t *dd, float *sd) __attribute__((always_inline)) {
    const int hq = hkv * a.G + tt / ntile_h;
    const int i0 = qlo + (tt % ntile_h) * ROWS;
    const size_t rowbase = ((size_t)b * a.Hq + hq) * a.Lq;
    if (lw < 0) return;
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
      const int blk = lw * BPL + i;
      const int row = blk * RPB + lane / CPR;
      const int c = (lane % CPR) ^ tswz<D>(row);
      const size_t grow = rowbase + min(i0 + row, a.Lq - 1);
      dma_to_lds<16>(a.q + grow * D + 8 * c, qd + blk * 512);
      dma_to_lds<16>(a.dout + grow * D + 8 * c, dd + blk * 512);
    }
    if (lw < 2) {
      const float *src = lw == 0 ? a.lse2 : a.delta;
      const size_t grow = rowbase + min(i0 + lane, a.Lq - 1);
      dma_to_lds<4>(src + grow, sd + ROWS * lw);
    }
  };
  auto wait_tile = [&](bool younger) __attribute__((always_inline)) {
    if (younger) {
      if (lw >= 0 && lw < 2) ATTN_BWD_WAIT_VM(2 * BPL + 1);
      else ATTN_BWD_WAIT_VM(2 * BPL);
    } else {
      ATTN_BWD_WAIT_VM(0);
    }
  };

  const float c = a.c;
  auto skip_half = [&](int i0h) __attribute__((always_inline)) {
    if (i0h >= a.Lq) return true;
    return a.causal && (i0h + 31 + off < kw0 || (win && i0h + off - win + 1 > kw0 + 31));
  };
  auto cross_half = [&](int i0h) __attribute__((always_inline)) {
    return i0h + 31 >= a.Lq || (a.causal && (i0h + off < kw0 + 31 || (win && i0h + 31 + off - win + 1 > kw0)));
  };
  // 8 MFMAs: acc16 = (rows of the half) x (the pair's keys), A from LDS rows
  auto rowprod = [&](const uint16_t *xt, f32x16 &r) __attribute__((always_inline)) {
    r = f32x16{};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      r = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ld16(xt + roff[ks])), kvf[ks], r, 0, 0, 0);
  };
  // acc^T += X^T Y (k = the half's 32 rows), X^T read transposed from LDS
  // (the half's two 16-row steps outermost, so that consecutive MFMAs go to
  // different accumulators; each accumulator keeps its order)
  auto colprod = [&](const uint16_t *xt, const bf16x8(&y)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int qh = 0; qh < 2; ++qh)
#pragma unroll
      for (int dd = 0; dd < D / 32; ++dd)
        acc[dd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            tr_operand(xt + 16 * qh * D + tlo[dd], xt + 16 * qh * D + thi[dd]), y[qh], acc[dd], 0, 0, 0);
  };
  auto pack16 = [&](const float(&v)[16], bf16x8(&o)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int qh = 0; qh < 2; ++qh)
      o[qh] = pack8(v[8 * qh], v[8 * qh + 1], v[8 * qh + 2], v[8 * qh + 3], v[8 * qh + 4], v[8 * qh + 5], v[8 * qh + 6],
                    v[8 * qh + 7]);
  };

  // One stage, for one role (the two roles run separate copies of the loop,
  // so that each keeps only its own values live; both pass the same
  // barriers, in the same number and order).
  auto step = [&](int tt, const uint16_t *qt, const uint16_t *dt, const float *st, uint16_t *qn, uint16_t *dn,
                  float *sn, auto role) __attribute__((always_inline)) {
    constexpr bool PW = decltype(role)::value;
    wait_tile(tt + 1 < ntile);
    barrier_keep_loads();
    if (ATTN_BWD_PAIR_LOADS != 2 && tt + 2 < ntile) issue(tt + 2, qn, dn, sn);
    const int i0 = qlo + (tt % ntile_h) * ROWS;
    bool live[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) live[h] = !skip_half(i0 + 32 * h);
    if constexpr (PW) {
      bf16x8 pk[2][2];      // P of each half, kept for dV
      // P of half h = exp2(S c - lse2), written to LDS for the partner
      auto pexp = [&](int h, const f32x16 &s, auto masked) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(masked)::value;
        float pv[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int r = 8 * (rr >> 2) + 4 * hh + (rr & 3);
          float pe = fast_exp2(__builtin_fmaf(s[rr], c, -st[32 * h + r]));
          if (MASKED) {
            const int i = i0 + 32 * h + r;
            const int lim = i + off;
            const bool vis = i < a.Lq && (!a.causal || (key <= lim && (!win || key > lim - win)));
            pe = vis ? pe : 0.f;
          }
          pv[rr] = pe;
        }
        float *pw = &pbuf[pair][h][0];
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<f32x4 *>(pw + 4 * (g * 64 + lane)) = f32x4{pv[4 * g], pv[4 * g + 1], pv[4 * g + 2], pv[4 * g + 3]};
      };
      constexpr int PPIPE = D == 64 ? ATTN_BWD_P_PIPE64 : ATTN_BWD_P_PIPE128;
      if (PPIPE > 0 && live[0] && live[1] && !cross_half(i0) && !cross_half(i0 + 32)) {
        // both halves unmasked: the first half's exponentials beside the
        // second half's S products
        f32x16 s0, s1;
        rowprod(qt, s0);
        sched_reads_ahead<D / 16, 1, kQkAhead<D>>();
        rowprod(qt + 32 * D, s1);
        pexp(0, s0, std::false_type{});
        sched_interleave<D / 16, 1, kQkAhead<D>, (PPIPE > 0 ? PPIPE : 1)>();
        pexp(1, s1, std::false_type{});
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (!live[h]) continue;
          f32x16 s;
          rowprod(qt + 32 * h * D, s);
          sched_reads_ahead<D / 16, 1, kQkAhead<D>>();
          // only halves that cross a mask boundary or the end of the rows evaluate the mask
          if (cross_half(i0 + 32 * h)) pexp(h, s, std::true_type{});
          else pexp(h, s, std::false_type{});
        }
      }
      barrier_keep_loads();   // P of every pair is in LDS
      // the bf16 packing of P for dV happens here, in the phase where this
      // wave has slack, from the copy it handed to its partner; so does the
      // staging of stage tt + 2 (into the buffers of stage tt - 1, free since
      // the stage's first barrier)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (live[h]) {
          {
            const float *pr = &pbuf[pair][h][0];
            float pv[16];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const f32x4 p4 = *reinterpret_cast<const f32x4 *>(pr + 4 * (g * 64 + lane));
#pragma unroll
              for (int i = 0; i < 4; ++i) pv[4 * g + i] = p4[i];
            }
            pack16(pv, pk[h]);
          }
          colprod(dt + 32 * h * D, pk[h]);
          sched_reads_ahead<2 * (D / 32), 2, kTrAhead<D>>();
        }
        if (ATTN_BWD_PAIR_LOADS == 2 && h == 0 && tt + 2 < ntile) issue(tt + 2, qn, dn, sn);
      }
    } else {
      f32x16 dp[2];         // dP of each half
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (!live[h]) continue;
        rowprod(dt + 32 * h * D, dp[h]);
        sched_reads_ahead<D / 16, 1, kQkAhead<D>>();
        // dP - delta here, where this wave has slack (the phase after the
        // barrier holds the stage's critical path)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) dp[h][rr] -= st[ROWS + 32 * h + 8 * (rr >> 2) + 4 * hh + (rr & 3)];
      }
      barrier_keep_loads();   // the partner's P is in LDS
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (!live[h]) continue;
        const float *pr = &pbuf[pair][h][0];
        float dsv[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 p4 = *reinterpret_cast<const f32x4 *>(pr + 4 * (g * 64 + lane));
#pragma unroll
          for (int i = 0; i < 4; ++i) dsv[4 * g + i] = p4[i] * dp[h][4 * g + i];
        }
        bf16x8 sk[2];
        pack16(dsv, sk);
        colprod(qt + 32 * h * D, sk);
        sched_reads_ahead<2 * (D / 32), 2, kTrAhead<D>>();
      }
    }
  };
  auto run = [&](auto role) __attribute__((always_inline)) {
    issue(0, qa, da, sa);
    if (ntile > 1) issue(1, qb, db_, sb);
    for (int tt = 0; tt < ntile; tt += 3) {
      step(tt, qa, da, sa, qc, dc, sc_, role);
      if (tt + 1 >= ntile) break;
      step(tt + 1, qb, db_, sb, qa, da, sa, role);
      if (tt + 2 >= ntile) break;
      step(tt + 2, qc, dc, sc_, qb, db_, sb, role);
    }
  };

  ATTN_BWD_WAIT_VM(0);
  if (ntile > 0) {
    if (pwave) run(std::true_type{});
    else run(std::false_type{});
  }

  // dk = scale dK (partners), dv = dV (P-waves); lane: key column, dims 32 dd + 8 j + 4 hh + (0..3)
  if (key < a.Lk) {
    uint16_t *op = (pwave ? a.dv : a.dk) + kvbase + (size_t)key * D;
    const float scl = pwave ? 1.f : a.scale;
#pragma unroll
    for (int dd = 0; dd < D / 32; ++dd)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 o4;
#pragma unroll
        for (int i = 0; i < 4; ++i) o4[i] = (__bf16)(acc[dd][4 * j + i] * scl);
        *reinterpret_cast<bf16x4 *>(op + 32 * dd + 8 * j + 4 * hh) = o4;
      }
  }
}

// ---------------------------------------------------------------------------
// dq
// ---------------------------------------------------------------------------
// keys per tile of the dq loop: 32 keeps a wave within 256 registers and a
// workgroup within 48 KiB of LDS (D <= 128), so two waves share each SIMD
#ifndef ATTN_BWD_DQ_BK
#define ATTN_BWD_DQ_BK 32
#endif
template <int D>
constexpr int kBwdQKeys = D == 256 ? 32 : ATTN_BWD_DQ_BK;
// waves per SIMD the dq kernel is built for (two need 32-key tiles: registers
// and LDS for two workgroups per CU)
template <int D>
constexpr int kBwdQWaves = (D <= 128 && kBwdQKeys<D> == 32) ? 2 : 1;

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kBwdQWaves<D>))) void bwd_dq_kernel(BackwardArgs a) {
  constexpr int CPR = D / 8;
  constexpr int BK = kBwdQKeys<D>;
  constexpr int TILE = BK * D;
  constexpr int RPB = 512 / D;                       // rows per 1 KiB direct load
  constexpr int BPW = TILE * 2 / 1024 / kBwdWaves;   // 1 KiB blocks per wave per tensor and tile
  static_assert(BPW * kBwdWaves * 1024 == TILE * 2, "tile must split evenly over the waves");
  // three stages of K and V tiles, each its own array
  __shared__ __attribute__((aligned(1024))) uint16_t ka[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t kb_[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t kc[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t va[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t vb[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t vc[TILE];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int ql = lane & 31, hh = lane >> 5, g16 = lane >> 4, j16 = lane & 15;

  // workgroup -> (row block, head group, b, hkv): waves are hpw heads x wph
  // row sub-blocks of 32 rows.  Row blocks in descending order (causal: the
  // rows that see the most keys start first), all heads of a row block
  // together.
  const int hpw = a.dq_hpw, wph = kBwdWaves / hpw;
  const int rows_wg = 32 * wph;
  const int nrb = (a.Lq + rows_wg - 1) / rows_wg;
  const int ngrp = a.G / hpw;
  const int nu = ngrp * a.Hkv * a.B;
  const int t = blockIdx.x;
  const int rbk = nrb - 1 - t / nu;
  int u = t % nu;
  const int grp = u % ngrp;
  u /= ngrp;
  const int hkv = u % a.Hkv;
  const int b = u / a.Hkv;
  const int hq = hkv * a.G + grp * hpw + w / wph;
  const int r0w = rbk * rows_wg + 32 * (w % wph);   // this wave's first row
  const int qrow = r0w + ql;                        // this lane's query row
  const int off = a.Lk - a.Lq;
  const int win = a.window;

  // q and dout rows as B operands: lane (ql, hh) holds row qrow, dims 16 ks + 8 hh
  const size_t rowi = ((size_t)b * a.Hq + hq) * a.Lq + (qrow < a.Lq ? qrow : 0);
  bf16x8 qf[D / 16], of[D / 16];
  {
    const u32x4 z = {0u, 0u, 0u, 0u};
    const bool in = qrow < a.Lq;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      qf[ks] = as_bf16x8(in ? ld16(a.q + rowi * D + 16 * ks + 8 * hh) : z);
      of[ks] = as_bf16x8(in ? ld16(a.dout + rowi * D + 16 * ks + 8 * hh) : z);
    }
  }
  const float lse2 = qrow < a.Lq ? a.lse2[rowi] : __builtin_inff();
  const float del = qrow < a.Lq ? a.delta[rowi] : 0.f;

  // key range of the workgroup's rows
  const int rlo = rbk * rows_wg, rhi = min(a.Lq, rlo + rows_wg) - 1;
  int kbeg = 0, kend = a.Lk;
  if (a.causal) {
    kend = min(a.Lk, rhi + off + 1);
    if (win) kbeg = max(0, rlo + off - win + 1);
  }
  const int jbeg = kbeg / BK;
  const int nt = kend > kbeg ? (kend + BK - 1) / BK - jbeg : 0;
  // this wave's key range (for skipping and masking)
  const int wlo = r0w, whi = min(a.Lq, r0w + 32) - 1;
  const int kend_w = a.causal ? min(a.Lk, whi + off + 1) : a.Lk;
  const int kbeg_w = (a.causal && win) ? max(0, wlo + off - win + 1) : 0;
  // keys from kfull on may be hidden from some row of the wave (or lie past Lk)
  const int kfull = a.causal ? min(a.Lk, wlo + off + 1) : a.Lk;
  const int klo_until = (a.causal && win) ? whi + off - win + 1 : 0;

  int roff[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) roff[ks] = toff<D>(ql, 2 * ks + hh);
  int tlo[D / 32], thi[D / 32];
  {
    const int r = 4 * hh + (j16 >> 2);
    const int c = 2 * (g16 & 1) + ((j16 & 3) >> 1);
#pragma unroll
    for (int dd = 0; dd < D / 32; ++dd) {
      tlo[dd] = toff<D>(r, 4 * dd + c) + 4 * (j16 & 1);
      thi[dd] = toff<D>(r + 8, 4 * dd + c) + 4 * (j16 & 1);
    }
  }

  f32x16 dq[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) dq[i] = f32x16{};

  // Tile jj of K and V straight from global memory into LDS (as the dk/dv
  // kernel stages q and dout); keys past the end are read from the last key
  // and masked.  Per tile a wave issues 2 BPW loads.
  const size_t kvrow = ((size_t)b * a.Hkv + hkv) * (size_t)a.Lk;   // first key row of this KV head
  auto issue = [&](int jj, uint16_t *kd, uint16_t *vd) __attribute__((always_inline)) {
    const int k0 = (jbeg + jj) * BK;
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int blk = wu * BPW + i;
      const int row = blk * RPB + lane / CPR;
      const int c = (lane % CPR) ^ tswz<D>(row);
      const size_t grow = kvrow + min(k0 + row, a.Lk - 1);
      dma_to_lds<16>(a.k + grow * D + 8 * c, kd + blk * 512);
      dma_to_lds<16>(a.v + grow * D + 8 * c, vd + blk * 512);
    }
  };

  const float c = a.c;
  auto compute = [&](int jj, const uint16_t *kt, const uint16_t *vt) __attribute__((always_inline)) {
    const int k0 = (jbeg + jj) * BK;
    if (uniform(k0 >= kend_w || k0 + BK <= kbeg_w)) return;
    f32x16 s[BK / 32], dp[BK / 32];
#pragma unroll
    for (int rb = 0; rb < BK / 32; ++rb) {
      s[rb] = f32x16{};
      dp[rb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        s[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ld16(kt + 32 * rb * D + roff[ks])), qf[ks], s[rb],
                                                        0, 0, 0);
        dp[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ld16(vt + 32 * rb * D + roff[ks])), of[ks],
                                                         dp[rb], 0, 0, 0);
      }
    }
    sched_reads_ahead<2 * (BK / 32) * (D / 16), 1, kQkAhead<D>>();
    // this lane: query row qrow, keys k0 + 32 rb + 8 (rr >> 2) + 4 hh + (rr & 3)
    const int lim = a.causal ? qrow + off : a.Lk - 1;
    bf16x8 sb[BK / 16];
    auto ds_tile = [&](auto masked) __attribute__((always_inline)) {
      constexpr bool MASKED = decltype(masked)::value;
#pragma unroll
      for (int rb = 0; rb < BK / 32; ++rb) {
        float dsv[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int kk = k0 + 32 * rb + 8 * (rr >> 2) + 4 * hh + (rr & 3);
          float pe = fast_exp2(__builtin_fmaf(s[rb][rr], c, -lse2));
          if (MASKED) {
            const bool vis = kk < a.Lk && kk <= lim && (!(a.causal && win) || kk > lim - win);
            pe = vis ? pe : 0.f;
          }
          dsv[rr] = pe * (dp[rb][rr] - del);
        }
        sb[2 * rb] = pack8(dsv[0], dsv[1], dsv[2], dsv[3], dsv[4], dsv[5], dsv[6], dsv[7]);
        sb[2 * rb + 1] = pack8(dsv[8], dsv[9], dsv[10], dsv[11], dsv[12], dsv[13], dsv[14], dsv[15]);
      }
    };
    // only tiles that cross the diagonal, a window edge or the end of the
    // keys evaluate the mask
    if (uniform(k0 + BK > kfull || k0 < klo_until)) ds_tile(std::true_type{});
    else ds_tile(std::false_type{});
    // dQ^T += K^T dS^T  (k = the tile's keys)
#pragma unroll
    for (int dd = 0; dd < D / 32; ++dd)
#pragma unroll
      for (int kc2 = 0; kc2 < BK / 16; ++kc2)
        dq[dd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            tr_operand(kt + 16 * kc2 * D + tlo[dd], kt + 16 * kc2 * D + thi[dd]), sb[kc2], dq[dd], 0, 0, 0);
    sched_reads_ahead<(D / 32) * (BK / 16), 2, kTrAhead<D>>();
  };
  auto step = [&](int jj, const uint16_t *kt, const uint16_t *vt, uint16_t *kn, uint16_t *vn)
      __attribute__((always_inline)) {
    if (jj + 1 < nt) ATTN_BWD_WAIT_VM(2 * BPW);
    else ATTN_BWD_WAIT_VM(0);
    barrier_keep_loads();
    if (jj + 2 < nt) issue(jj + 2, kn, vn);
    compute(jj, kt, vt);
  };

  // the q/dout operand loads complete before any staged load is issued (see
  // the dk/dv kernel)
  ATTN_BWD_WAIT_VM(0);
  if (nt > 0) {
    issue(0, ka, va);
    if (nt > 1) issue(1, kb_, vb);
    for (int jj = 0; jj < nt; jj += 3) {
      step(jj, ka, va, kc, vc);
      if (jj + 1 >= nt) break;
      step(jj + 1, kb_, vb, ka, va);
      if (jj + 2 >= nt) break;
      step(jj + 2, kc, vc, kb_, vb);
    }
  }

  if (qrow < a.Lq) {
    uint16_t *qp = a.dq + rowi * D;
    const float scl = a.scale;
#pragma unroll
    for (int dd = 0; dd < D / 32; ++dd)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 v4;
#pragma unroll
        for (int i = 0; i < 4; ++i) v4[i] = (__bf16)(dq[dd][4 * j + i] * scl);
        *reinterpret_cast<bf16x4 *>(qp + 32 * dd + 8 * j + 4 * hh) = v4;
      }
  }
}

// dq with two groups of waves (D = 64, 128): eight waves, wave w and wave
// w + 4 on one SIMD, each owning 32 query rows as in bwd_dq_kernel.  Per
// 32-key tile j the matrix work G(j) = [dQ += K(j-1)^T dS(j-1)^T,
// S^T(j) = K(j) Q^T, dP^T(j) = V(j) dO^T] and the vector work
// dS(j) = P(j) (dP(j) - delta) alternate between the groups inside one step:
// group A (waves 0-3) runs G(j) and then dS(j), group B runs dS(j-1) and then
// G(j), so the exponentials of one wave execute beside the MFMAs of its SIMD
// neighbour (as in the forward's ping-pong).  K and V tiles sit in a ring of
// four LDS stages (tile j-1 is still read by dQ in step j); group A's waves
// load tile j+2 in step j, among their S / dP MFMAs.  Same products in the
// same order per accumulator as bwd_dq_kernel (bit-identical).
template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dq2_kernel(BackwardArgs a) {
  constexpr int NW = 8;
  constexpr int CPR = D / 8;
  constexpr int BK = 32;
  constexpr int TILE = BK * D;
  constexpr int RPB = 512 / D;                       // rows per 1 KiB direct load
  constexpr int NB = TILE * 2 / 1024;                // 1 KiB blocks per tensor and tile
  constexpr int NL = NB < NW / 2 ? NB : NW / 2;      // waves that load (group A's first NL)
  constexpr int BPL = NB / NL;                       // their blocks per tensor and tile
  static_assert(BPL * NL == NB, "tile must split evenly over the loading waves");
  __shared__ __attribute__((aligned(1024))) uint16_t kst[4][TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t vst[4][TILE];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const bool grpA = wu < NW / 2;
  const int lw = wu < NL ? wu : -1;                  // index among the loading waves (< 0: none)
  const int ql = lane & 31, hh = lane >> 5, g16 = lane >> 4, j16 = lane & 15;

  // workgroup -> (row block, head group, b, hkv); waves are hpw heads x wph
  // row sub-blocks of 32 rows; row blocks in descending order
  const int hpw = a.dq_hpw, wph = NW / hpw;
  const int rows_wg = 32 * wph;
  const int nrb = (a.Lq + rows_wg - 1) / rows_wg;
  const int ngrp = a.G / hpw;
  const int nu = ngrp * a.Hkv * a.B;
  const int t = blockIdx.x;
  const int rbk = nrb - 1 - t / nu;
  int u = t % nu;
  const int grp = u % ngrp;
  u /= ngrp;
  const int hkv = u % a.Hkv;
  const int b = u / a.Hkv;
  const int hq = hkv * a.G + grp * hpw + wu / wph;
  const int r0w = rbk * rows_wg + 32 * (wu % wph);
  const int qrow = r0w + ql;
  const int off = a.Lk - a.Lq;
  const int win = a.window;

  const size_t rowi = ((size_t)b * a.Hq + hq) * a.Lq + (qrow < a.Lq ? qrow : 0);
  bf16x8 qf[D / 16], of[D / 16];
  {
    const u32x4 z = {0u, 0u, 0u, 0u};
    const bool in = qrow < a.Lq;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      qf[ks] = as_bf16x8(in ? ld16(a.q + rowi * D + 16 * ks + 8 * hh) : z);
      of[ks] = as_bf16x8(in ? ld16(a.dout + rowi * D + 16 * ks + 8 * hh) : z);
    }
  }
  const float lse2 = qrow < a.Lq ? a.lse2[rowi] : __builtin_inff();
  const float del = qrow < a.Lq ? a.delta[rowi] : 0.f;

  // key range of the workgroup's rows (every wave walks it: one barrier per tile)
  const int rlo = rbk * rows_wg, rhi = min(a.Lq, rlo + rows_wg) - 1;
  int kbeg = 0, kend = a.Lk;
  if (a.causal) {
    kend = min(a.Lk, rhi + off + 1);
    if (win) kbeg = max(0, rlo + off - win + 1);
  }
  const int jbeg = kbeg / BK;
  const int nt = kend > kbeg ? (kend + BK - 1) / BK - jbeg : 0;
  // this wave's key range (tiles outside it are skipped by the wave)
  const int wlo = r0w, whi = min(a.Lq, r0w + 32) - 1;
  const int kend_w = a.causal ? min(a.Lk, whi + off + 1) : a.Lk;
  const int kbeg_w = (a.causal && win) ? max(0, wlo + off - win + 1) : 0;
  const int kfull = a.causal ? min(a.Lk, wlo + off + 1) : a.Lk;
  const int klo_until = (a.causal && win) ? whi + off - win + 1 : 0;

  int roff[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) roff[ks] = toff<D>(ql, 2 * ks + hh);
  int tlo[D / 32], thi[D / 32];
  {
    const int r = 4 * hh + (j16 >> 2);
    const int c = 2 * (g16 & 1) + ((j16 & 3) >> 1);
#pragma unroll
    for (int dd = 0; dd < D / 32; ++dd) {
      tlo[dd] = toff<D>(r, 4 * dd + c) + 4 * (j16 & 1);
      thi[dd] = toff<D>(r + 8, 4 * dd + c) + 4 * (j16 & 1);
    }
  }

  f32x16 dq[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) dq[i] = f32x16{};

  const size_t kvrow = ((size_t)b * a.Hkv + hkv) * (size_t)a.Lk;
  auto issue = [&](int jj, uint16_t *kd, uint16_t *vd) __attribute__((always_inline)) {
    if (lw < 0) return;
    const int k0 = (jbeg + jj) * BK;
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
      const int blk = lw * BPL + i;
      const int row = blk * RPB + lane / CPR;
      const int c = (lane % CPR) ^ tswz<D>(row);
      const size_t grow = kvrow + min(k0 + row, a.Lk - 1);
      dma_to_lds<16>(a.k + grow * D + 8 * c, kd + blk * 512);
      dma_to_lds<16>(a.v + grow * D + 8 * c, vd + blk * 512);
    }
  };
  auto active = [&](int jj) __attribute__((always_inline)) {
    const int k0 = (jbeg + jj) * BK;
    return jj >= 0 && jj < nt && !uniform(k0 >= kend_w || k0 + BK <= kbeg_w);
  };

  const float c = a.c;
  // dS^T = P (dP - delta) of tile jj from its S^T and dP^T, packed for dQ
  auto ds_tile = [&](int jj, const f32x16 &s, const f32x16 &dp, bf16x8(&sb)[2]) __attribute__((always_inline)) {
    const int k0 = (jbeg + jj) * BK;
    const int lim = a.causal ? qrow + off : a.Lk - 1;
    auto body = [&](auto masked) __attribute__((always_inline)) {
      constexpr bool MASKED = decltype(masked)::value;
      float dsv[16];
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int kk = k0 + 8 * (rr >> 2) + 4 * hh + (rr & 3);
        float pe = fast_exp2(__builtin_fmaf(s[rr], c, -lse2));
        if (MASKED) {
          const bool vis = kk < a.Lk && kk <= lim && (!(a.causal && win) || kk > lim - win);
          pe = vis ? pe : 0.f;
        }
        dsv[rr] = pe * (dp[rr] - del);
      }
      sb[0] = pack8(dsv[0], dsv[1], dsv[2], dsv[3], dsv[4], dsv[5], dsv[6], dsv[7]);
      sb[1] = pack8(dsv[8], dsv[9], dsv[10], dsv[11], dsv[12], dsv[13], dsv[14], dsv[15]);
    };
    if (uniform(k0 + BK > kfull || k0 < klo_until)) body(std::true_type{});
    else body(std::false_type{});
  };
  // dQ^T += K^T dS^T of the tile in stage kp (K^T read transposed)
  auto dq_part = [&](const uint16_t *kp, const bf16x8(&sb)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int kc2 = 0; kc2 < BK / 16; ++kc2)
#pragma unroll
      for (int dd = 0; dd < D / 32; ++dd)
        dq[dd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            tr_operand(kp + 16 * kc2 * D + tlo[dd], kp + 16 * kc2 * D + thi[dd]), sb[kc2], dq[dd], 0, 0, 0);
    sched_reads_ahead<(D / 32) * (BK / 16), 2, kTrAhead<D>>();
  };
  // S^T = K Q^T and dP^T = V dO^T of the tile in stages kt, vt; NLD > 0: the
  // direct loads `loads` (NLD of them) go among the MFMAs, one every SP
  auto sdp_part = [&](const uint16_t *kt, const uint16_t *vt, f32x16 &s, f32x16 &dp, auto loads, auto nld)
      __attribute__((always_inline)) {
    constexpr int NLD = decltype(nld)::value;
    s = f32x16{};
    dp = f32x16{};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ld16(kt + roff[ks])), qf[ks], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ld16(vt + roff[ks])), of[ks], dp, 0, 0, 0);
    }
    loads();
    constexpr int N = 2 * (D / 16);
    constexpr int AH = kQkAhead<D>;
    constexpr int SP = NLD > 0 && N / (NLD > 0 ? NLD : 1) > 0 ? N / (NLD > 0 ? NLD : 1) : 1;
    __builtin_amdgcn_sched_group_barrier(0x100, AH, 0);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (NLD > 0 && i % SP == 0 && i / SP < NLD) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
      if (i < N - AH) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };
  auto none = []() __attribute__((always_inline)) {};
  // Values carried from one step to the next: group A the packed dS^T of its
  // last tile, group B the S^T and dP^T of its last tile.  Every path through
  // a step writes them (zeros for a tile the wave skips), so that they are
  // not held live through the parts of the step that do not need them.
  bf16x8 sbc[2];
  f32x16 sc, dpc;
  // step jj, tile jj in stage P = jj % 4: tile jj's loads are complete (the
  // loads issued in step jj-1 may be in flight); the barrier publishes them
  // and frees stage (P + 2) % 4 (tile jj-2), into which group A's waves load
  // tile jj+2 among their S / dP MFMAs (past the last tile: a repeat of it,
  // never read), so every step issues the same loads and waits for the same
  // count
  auto step = [&](int jj, auto stage, auto role) __attribute__((always_inline)) {
    constexpr int P = decltype(stage)::value;
    constexpr bool A = decltype(role)::value;
    if (lw >= 0) ATTN_BWD_WAIT_VM(2 * BPL);
    barrier_keep_loads();
    const bool ap = active(jj - 1), ac = active(jj);
    const uint16_t *kp = kst[(P + 3) & 3];
    if constexpr (A) {
      // G(jj), then dS(jj); the S / dP products run on every step for the
      // loads among them (a tile this wave does not see gives dS = 0)
      __builtin_amdgcn_s_setprio(1);
      if (ap) dq_part(kp, sbc);
      f32x16 s, dp;
      if (lw >= 0) {
        sdp_part(kst[P], vst[P], s, dp, [&]() __attribute__((always_inline)) {
          issue(min(jj + 2, nt - 1), kst[(P + 2) & 3], vst[(P + 2) & 3]);
        }, std::integral_constant<int, 2 * BPL>{});
      } else if (ac) {
        sdp_part(kst[P], vst[P], s, dp, none, std::integral_constant<int, 0>{});
      }
      __builtin_amdgcn_s_setprio(0);
      if (ac) {
        ds_tile(jj, s, dp, sbc);
      } else {
        sbc[0] = bf16x8{};
        sbc[1] = bf16x8{};
      }
    } else {
      // dS(jj-1), then G(jj)
      if (ap) {
        bf16x8 sb[2];
        ds_tile(jj - 1, sc, dpc, sb);
        __builtin_amdgcn_s_setprio(1);
        dq_part(kp, sb);
      } else {
        __builtin_amdgcn_s_setprio(1);
      }
      if (ac) {
        sdp_part(kst[P], vst[P], sc, dpc, none, std::integral_constant<int, 0>{});
      } else {
        sc = f32x16{};
        dpc = f32x16{};
      }
      __builtin_amdgcn_s_setprio(0);
    }
  };
  // the two groups run separate copies of the loop (each keeps only its own
  // values live); both pass the same barriers in the same number
  auto run = [&](auto role) __attribute__((always_inline)) {
    issue(0, kst[0], vst[0]);
    issue(min(1, nt - 1), kst[1], vst[1]);
    for (int jj = 0; jj <= nt; jj += 4) {
      step(jj, std::integral_constant<int, 0>{}, role);
      if (jj + 1 > nt) break;
      step(jj + 1, std::integral_constant<int, 1>{}, role);
      if (jj + 2 > nt) break;
      step(jj + 2, std::integral_constant<int, 2>{}, role);
      if (jj + 3 > nt) break;
      step(jj + 3, std::integral_constant<int, 3>{}, role);
    }
  };

  // the q/dout operand loads complete before any staged load is issued
  ATTN_BWD_WAIT_VM(0);
  if (nt > 0) {
    if (grpA) run(std::true_type{});
    else run(std::false_type{});
    ATTN_BWD_WAIT_VM(0);   // the repeats of the last tile have landed
  }

  if (qrow < a.Lq) {
    uint16_t *qp = a.dq + rowi * D;
    const float scl = a.scale;
#pragma unroll
    for (int dd = 0; dd < D / 32; ++dd)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 v4;
#pragma unroll
        for (int i = 0; i < 4; ++i) v4[i] = (__bf16)(dq[dd][4 * j + i] * scl);
        *reinterpret_cast<bf16x4 *>(qp + 32 * dd + 8 * j + 4 * hh) = v4;
      }
  }
}

// The dq kernel does not depend on the dk/dv kernel (both read only q, k, v,
// dout and the pre-pass's row statistics), so with ATTN_BWD_SIDE it runs on a
// second stream of the library, forked from and joined back into the caller's
// stream with events: its workgroups fill the CUs that the dk/dv kernel's
// last, uneven round leaves idle.  One side stream and event pair per device,
// created on first use; the fork and join are enqueued under a lock, so
// concurrent calls on one device share the side stream in order.
#ifndef ATTN_BWD_SIDE
#define ATTN_BWD_SIDE 1
#endif
namespace {
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
SideStream g_side[64];
std::mutex g_side_mu;
}  // namespace

template <int D>
static hipError_t launch_dq(const BackwardArgs &a, hipStream_t s) {
  if (ATTN_BWD_DQ_PAIRS && D <= 128) {
    BackwardArgs a2 = a;
    a2.dq_hpw = a.G % 8 == 0 ? 8 : a.dq_hpw;   // query heads per workgroup: divides G and 8
    const int rows_wg = 32 * (8 / a2.dq_hpw);
    const long long nrb = (a.Lq + rows_wg - 1) / rows_wg;
    hipLaunchKernelGGL((bwd_dq2_kernel<D <= 128 ? D : 128>), dim3((unsigned)(nrb * (a.G / a2.dq_hpw) * a.Hkv * a.B)),
                       dim3(512), 0, s, a2);
    return hipGetLastError();
  }
  const int rows_wg = 32 * (kBwdWaves / a.dq_hpw);
  const long long nrb = (a.Lq + rows_wg - 1) / rows_wg;
  hipLaunchKernelGGL((bwd_dq_kernel<D>), dim3((unsigned)(nrb * (a.G / a.dq_hpw) * a.Hkv * a.B)), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_dkdv(const BackwardArgs &a, hipStream_t s) {
  const long long nkb = (a.Lk + kBwdKeys - 1) / kBwdKeys;
  if (ATTN_BWD_PAIRS && D <= 128)
    hipLaunchKernelGGL((bwd_dkdv2_kernel<D <= 128 ? D : 128>), dim3((unsigned)(nkb * a.B * a.Hkv)), dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<D>), dim3((unsigned)(nkb * a.B * a.Hkv)), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_bwd_t(const BackwardArgs &a, hipStream_t s) {
  const long long rows = (long long)a.B * a.Hq * a.Lq;
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int dev = -1;
  if (!ATTN_BWD_SIDE || hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    if ((e = launch_dkdv<D>(a, s)) != hipSuccess) return e;
    return launch_dq<D>(a, s);
  }
  std::lock_guard<std::mutex> lk(g_side_mu);
  SideStream &ss = g_side[dev];
  if (ss.s == nullptr) {
    SideStream n;
    if ((e = hipStreamCreateWithFlags(&n.s, hipStreamNonBlocking)) == hipSuccess &&
        (e = hipEventCreateWithFlags(&n.fork, hipEventDisableTiming)) == hipSuccess &&
        (e = hipEventCreateWithFlags(&n.join, hipEventDisableTiming)) == hipSuccess) {
      ss = n;
    } else {
      if (n.fork) (void)hipEventDestroy(n.fork);
      if (n.s) (void)hipStreamDestroy(n.s);
      return e;
    }
  }
  // fork after the pre-pass, whose row statistics the dq kernel reads
  if ((e = hipEventRecord(ss.fork, s)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(ss.s, ss.fork, 0)) != hipSuccess) return e;
  if ((e = launch_dq<D>(a, ss.s)) != hipSuccess) return e;
  if ((e = hipEventRecord(ss.join, ss.s)) != hipSuccess) return e;
  if ((e = launch_dkdv<D>(a, s)) != hipSuccess) return e;
  return hipStreamWaitEvent(s, ss.join, 0);
}

int backward_dq_heads(int G) {
  return G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1);
}

hipError_t launch_backward(const BackwardArgs &a, int D, hipStream_t s) {
  switch (D) {
    case 64: return launch_bwd_t<64>(a, s);
    case 128: return launch_bwd_t<128>(a, s);
    case 256: return launch_bwd_t<256>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
