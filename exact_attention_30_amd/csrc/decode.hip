// Decode: one new query row per sequence (all G query heads of a KV head)
// over a ragged KV cache, split along the keys, then merged.
//
// Method (pages, by title): "어텐션 구현 고르기, SDPA·FlashAttention 메모리와
// GPU 비용", section "is_causal 마스크 정렬, KV 캐시와 쓸 때의 함정" (the new
// token's K/V are in the cache; one query attends to every cached key with no
// mask) and section "KV 캐시를 끄면 생기는 일, use_cache 비용" (cached K/V do
// not change); "Как NVIDIA учит нейросети думать быстрее…", section "Prefill и
// decode — это две разные задачи" (decode reads the whole cache per token and
// is bound by memory), section on group size (the G heads of a group share
// one read of K/V), section on parallelism (KV split into parts whose partial
// results are merged).
//
// Merge identity for disjoint key chunks c with normalised partial outputs
// o_c and log-sum-exps l_c: lse = log sum_c exp(l_c), out = sum_c
// exp(l_c - lse) o_c (it follows from splitting the softmax sum).
//
// gfx950 design
//  * Balanced flat split.  A one-workgroup planner kernel turns the device-side
//    lengths into a prefix sum of 32-key blocks per sequence.  The main kernel
//    runs exactly W persistent wave64 workgroups (one per resident wave slot);
//    the key blocks of all (sequence, KV head) segments, laid end to end, are
//    cut into W equal ranges, one per wave.  A wave streams its range once, for
//    all G query heads of each segment together, and writes one partial
//    (normalised O, lse) per segment piece it covers -- or the final output
//    when its piece is the whole segment.  Every wave does the same amount of
//    work whatever the length mix, nothing is launched for empty chunks, and
//    there are at most W + (number of segments) partials.
//  * S^T = K Q^T with v_mfma_f32_16x16x32_bf16: keys on the M side (16 per
//    block, two blocks per 32-key step), up to 16 query heads on the N side per
//    column block.  K rows are loaded straight from HBM into the A-operand
//    registers (64 contiguous bytes per lane), no LDS.
//  * K and V (or their int8 codes) are read with raw buffer loads over the
//    readable rows of a segment: keys outside them read as zeros, so a load
//    needs no select, and its offset is one per-lane register per block plus
//    the instruction's immediate (no 64-bit address arithmetic per load).
//  * V rows go to a per-wave LDS tile as loaded (16-byte writes, rows padded
//    by 32 bytes against bank conflicts); the V^T operand of O^T += V^T P^T
//    comes back with ds_read_b64_tr_b16 in the key order of P^T, which is
//    taken directly from the S^T accumulators.
//  * The next 32-key block's K and V loads are issued before the current
//    block is computed (two register sets, 16 KiB per wave in flight; one set
//    for D = 256 or four query-column blocks, where a second would spill).
//  * int8 caches (q8_0-style: one binary16 scale per 32-element block of a
//    row, element = scale * code rounded to bf16): the same kernel with the
//    codes loaded instead of bf16 rows, each block's scale rows in one load per
//    lane handed out through LDS, and the codes turned into the bf16 MFMA
//    operands in registers once they arrive.
//  * Lazy max update as in the prefill kernel.
//  * Wide row groups (33 to 64 query rows per KV head, bf16 caches, large
//    caches) take decode_wide_kernel instead: the same split and partials,
//    with two 32-row blocks per wave on v_mfma_f32_32x32x16_bf16 (row
//    statistics lane-local), and K/V moved to LDS by direct loads (two
//    blocks in flight without registers) and read as in the prefill kernel.
//  * The combine kernel (one wave per query row) merges the partials of the
//    segments that were split between waves.
#include "common.h"
#include "kernels.h"

// Load choices (compile-time):
//  ATTN_DEC_KNT / ATTN_DEC_VNT   nontemporal (streaming) loads for K / V
//  (K operand layout: lane group g, step ks holds dims 32 ks + 8 g, so that
//  each load instruction reads 64 contiguous bytes per key row)
#ifndef ATTN_DEC_KNT
#define ATTN_DEC_KNT 1
#endif
#ifndef ATTN_DEC_VNT
#define ATTN_DEC_VNT 1
#endif

namespace attn {

// Which wave's range contains flat block x, for the balanced split of `total`
// blocks over W waves (the first total % W waves take one block more).
ATTN_DEV long long wave_of(long long x, long long total, long long W) {
  const long long q = total / W, rem = total % W;
  const long long big = (q + 1) * rem;
  if (x < big) return x / (q + 1);
  return rem + (x - big) / q;
}

// First key of sequence b's segment: with a window, the earliest key any of
// its T rows sees, rounded down to a 32-key block; else 0.
ATTN_DEV int seg_begin(const DecodeArgs &a, int n) {
  return a.window ? (max(0, n - a.T - a.window + 1) & ~31) : 0;
}
ATTN_DEV long long seg_blocks(const DecodeArgs &a, int b) {
  const int n = max(0, min(a.lens[b], a.Lmax));
  return (n - seg_begin(a, n) + 31) / 32;
}

// Planner: pre[b] = sum over b' < b of the key blocks of sequence b'
// (ceil((n - first key) / 32)), pre[B] = the total.  One workgroup of 1024
// threads; each thread owns a contiguous slice of sequences.
__global__ __launch_bounds__(1024) void decode_plan_kernel(DecodeArgs a) {
  __shared__ long long part[1024];
  const int t = threadIdx.x;
  const int per = (a.B + 1023) / 1024;
  const int b0 = min(a.B, t * per), b1 = min(a.B, b0 + per);
  long long sum = 0;
  for (int b = b0; b < b1; ++b) sum += seg_blocks(a, b);
  part[t] = sum;
  __syncthreads();
  // inclusive scan of the 1024 slice sums (Hillis-Steele)
  for (int sh = 1; sh < 1024; sh <<= 1) {
    const long long v = t >= sh ? part[t - sh] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  long long run = part[t] - sum;  // exclusive prefix of this slice
  for (int b = b0; b < b1; ++b) {
    a.pre[b] = run;
    run += seg_blocks(a, b);
  }
  if (t == 1023) a.pre[a.B] = part[1023];
}

// int8 -> bf16 for 8 codes (two dwords) of one 32-element block with scale s:
// the codes are biased to unsigned bytes (xor 0x80), converted exactly, and
// x = s * (u - 128) is rounded to bf16 (nearest even).
ATTN_DEV u32x4 dequant8(uint32_t lo, uint32_t hi, float s) {
  const uint32_t a = lo ^ 0x80808080u, b = hi ^ 0x80808080u;
  const float o = -128.f * s;
  const bf16x8 r = pack8(__builtin_fmaf((float)(a & 0xffu), s, o), __builtin_fmaf((float)((a >> 8) & 0xffu), s, o),
                         __builtin_fmaf((float)((a >> 16) & 0xffu), s, o), __builtin_fmaf((float)(a >> 24), s, o),
                         __builtin_fmaf((float)(b & 0xffu), s, o), __builtin_fmaf((float)((b >> 8) & 0xffu), s, o),
                         __builtin_fmaf((float)((b >> 16) & 0xffu), s, o), __builtin_fmaf((float)(b >> 24), s, o));
  return __builtin_bit_cast(u32x4, r);
}
ATTN_DEV float half_bits_to_float(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// head dims (bit mask: 1 = D 64, 2 = D 128) for which wide row groups may
// take decode_wide_kernel (D = 256 would spill its registers)
#ifndef ATTN_DEC_WIDE
#define ATTN_DEC_WIDE 3
#endif
// Largest column-block count that keeps two register sets of K/V in flight.
#ifndef ATTN_DEC_DBUF_NCB
#define ATTN_DEC_DBUF_NCB 2
#endif

// Registers of one 32-key block in flight: bf16 K operands and V rows, or
// (Q8) the int8 codes and scales they are dequantized from.
template <int D, bool Q8>
struct DecodeRaw;
template <int D>
struct DecodeRaw<D, false> {
  static constexpr int KST = D / 32, VU = (D / 2 + 63) / 64;
  u32x4 kr[2 * KST];
  u32x4 vr[VU][8];
};
template <int D>
struct DecodeRaw<D, true> {
  // K: piece i of a lane in group g holds the 16 codes of dims 64 i + 16 g ...,
  // all inside one 32-element block (2 i + g / 2)
  static constexpr int KQ = D / 64;
  static constexpr int VU = (D / 2 + 63) / 64;
  static constexpr int SW = D / 64;   // dwords of one row's D/32 binary16 scales
  u32x4 kq[2][KQ];
  u32x2 vq[VU][8];
  // the block's scale rows, one per lane: lanes 0..31 the K rows of keys
  // kb + lane, lanes 32..63 the V rows of keys kb + lane - 32
  uint32_t sc[SW];
};

// One query-column block: two waves per SIMD (256 registers each); more
// column blocks need the whole register file.
template <int D, int NCB, bool Q8>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(NCB == 1 ? 2 : 1))) void decode_main_kernel(DecodeArgs a) {
  constexpr int KST = D / 32;            // 32-dim MFMA steps over the head dim
  constexpr int NKR = 2 * KST;           // K registers (16 B each) per 32-key block
  constexpr int VUN = D / 2;             // (8 keys x 8 dims) units per 32-key block
  constexpr int VU = (VUN + 63) / 64;    // units per lane
  // the block's V rows as loaded, row stride D + 16 (a 32-byte pad, so that
  // the 8 rows one half-wave's transposing read touches sit on 8 distinct
  // bank groups)
  constexpr int VRS = D + 16;
  __shared__ __attribute__((aligned(16))) uint16_t vt[32 * VRS];
  // int8 caches: the block's K and V scale rows ([2][32 keys][D / 32] binary16)
  __shared__ __attribute__((aligned(16))) uint16_t sct[Q8 ? 2 * 32 * (D / 32) : 2];

  const int lane = threadIdx.x;
  const int ql = lane & 15, g = lane >> 4;
  const long long W = gridDim.x, w = blockIdx.x;
  const long long HH = (long long)a.Hkv * a.n_hg;
  const long long total = a.pre[a.B] * HH;  // key blocks of all segments
  const long long q = total / W, rem = total % W;
  long long r = q * w + min(w, rem);
  const long long r1 = r + q + (w < rem ? 1 : 0);
  if (r >= r1) return;

  // segment holding block r: the largest b with HH * pre[b] <= r
  int b;
  {
    int lo = 0, hi = a.B;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (HH * a.pre[mid] <= r) lo = mid;
      else hi = mid;
    }
    b = lo;
  }
  long long nb = a.pre[b + 1] - a.pre[b];
  long long off = r - HH * a.pre[b];
  int hh = (int)(off / nb);
  long long blk = off - hh * nb;

  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  const float cexp = a.c;
  const bool cpos = cexp >= 0.f;
  const float maskval = cpos ? -__builtin_inff() : __builtin_inff();
  const int GT = a.G * a.T;               // query rows of one KV head
  const int GW = min(GT, decode_group(D));

  while (r < r1) {
    const long long take = min(nb - blk, r1 - r);
    const int hkv = hh / a.n_hg, hg = hh - hkv * a.n_hg;
    const int gq0 = hg * decode_group(D);
    const int gcnt = min(decode_group(D), GT - gq0);
    const int n = max(0, min(a.lens[b], a.Lmax));
    const int kseg = seg_begin(a, n);
    const int kmin = a.window ? max(0, n - a.T - a.window + 1) : 0;   // keys below are never read
    const int k0 = kseg + (int)(blk * 32);
    const int k1 = min(n, kseg + (int)((blk + take) * 32));
    const bool whole = (blk == 0) && (take == nb);
    // causal limit of this lane's query row in each column block: with T new
    // rows at the end of the cache, row t sees keys [0, n - T + t]
    // (and with a window, keys [n - T + t - window + 1, ...])
    int kcol[NCB], klo[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      kcol[cb] = n - a.T + 1 + (gq0 + 16 * cb + ql) % a.T;
      klo[cb] = a.window ? kcol[cb] - a.window : -0x7fffffff;
    }
    const int kfull = min(k1, n - a.T + 1);                      // keys below: below every row's limit
    const int klo_all = a.window ? n - a.window : -0x7fffffff;   // keys from here: above every row's start
    const long long slot = (long long)b * HH + hh + w;

    bf16x8 qf[NCB][KST];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int qi = 16 * cb + ql;
      // rows of a KV head are contiguous: (head g, position t) -> g * T + t
      const uint16_t *qp = a.q + (((size_t)b * a.Hq + hkv * a.G) * a.T + gq0 + min(qi, gcnt - 1)) * D;
#pragma unroll
      for (int ks = 0; ks < KST; ++ks)
        qf[cb][ks] = as_bf16x8(qi < gcnt ? ld16(qp + (Q8 ? 64 * (ks >> 1) + 16 * g + 8 * (ks & 1) : 32 * ks + 8 * g))
                                         : zero4);
    }
    const size_t base = ((size_t)b * a.Hkv + hkv) * (size_t)a.Lmax * D;
    const uint16_t *kg = a.kc + base;
    const uint16_t *vg = a.vc + base;

    f32x4 o[NCB][D / 16];
    float m_run[NCB], l_run[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      m_run[cb] = -__builtin_inff();
      l_run[cb] = 0.f;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) o[cb][db] = f32x4{};
    }

    using Raw = DecodeRaw<D, Q8>;
    const int8_t *kq8 = reinterpret_cast<const int8_t *>(a.kc) + base;
    const int8_t *vq8 = reinterpret_cast<const int8_t *>(a.vc) + base;
    const uint16_t *ksg = Q8 ? a.kscale + base / 32 : nullptr;
    const uint16_t *vsg = Q8 ? a.vscale + base / 32 : nullptr;
    const uint32_t zero2 = 0u;
#if ATTN_DEVICE_PASS
    // Buffer resources over this segment's readable rows [kmin, k1): a key
    // outside them gets an offset at or past the resource's end (keys below
    // kmin wrap to offsets near 2^32), and such loads return zeros without
    // touching memory.  Offsets: a per-lane constant plus (kb - kmin) rows
    // per block; the step within a block is the instruction's immediate.
    constexpr int EB = Q8 ? 1 : 2;   // bytes per cached element
    const auto rk = buf_rsrc(reinterpret_cast<const char *>(Q8 ? (const void *)kq8 : (const void *)kg) +
                                 (size_t)kmin * D * EB,
                             (uint32_t)(k1 - kmin) * (D * EB));
    const auto rv = buf_rsrc(reinterpret_cast<const char *>(Q8 ? (const void *)vq8 : (const void *)vg) +
                                 (size_t)kmin * D * EB,
                             (uint32_t)(k1 - kmin) * (D * EB));
    auto load = [&](Raw &raw, int kb) {
      const int rowb = (kb - kmin) * (D * EB);   // byte offset of the block's first key
      if constexpr (Q8) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const int vo = rowb + (16 * rb + ql) * D + 16 * g;
#pragma unroll
          for (int i = 0; i < Raw::KQ; ++i) raw.kq[rb][i] = __builtin_amdgcn_raw_buffer_load_b128(rk, vo + 64 * i, 0, 2);
        }
        {
          const int key = kb + (lane & 31);
          const bool in = key < k1 && key >= kmin;
          const uint16_t *ps = (lane < 32 ? ksg : vsg) + (size_t)(in ? key : kmin) * (D / 32);
          if constexpr (Raw::SW == 1) {
            raw.sc[0] = in ? __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(ps)) : 0u;
          } else if constexpr (Raw::SW == 2) {
            const u32x2 v2 =
                in ? __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(ps)) : u32x2{zero2, zero2};
            raw.sc[0] = v2[0];
            raw.sc[1] = v2[1];
          } else {
            const u32x4 v4 = in ? ld16_stream(ps) : zero4;
#pragma unroll
            for (int j = 0; j < 4; ++j) raw.sc[j] = v4[j];
          }
        }
#pragma unroll
        for (int iu = 0; iu < VU; ++iu) {
          const int u = lane + 64 * iu;
          if (VUN % 64 == 0 || u < VUN) {
            const int c = u % (D / 8), gg = u / (D / 8);
            const int v0 = rowb + 4 * gg * D + 8 * c, v1 = v0 + 16 * D;
#pragma unroll
            for (int kk = 0; kk < 8; ++kk)
              raw.vq[iu][kk] = __builtin_amdgcn_raw_buffer_load_b64(rv, (kk < 4 ? v0 : v1) + (kk & 3) * D, 0, 2);
          }
        }
      } else {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const int vo = rowb + (16 * rb + ql) * (D * 2) + 16 * g;
#pragma unroll
          for (int ks = 0; ks < KST; ++ks)
            raw.kr[rb * KST + ks] = __builtin_amdgcn_raw_buffer_load_b128(rk, vo + 64 * ks, 0, ATTN_DEC_KNT ? 2 : 0);
        }
#pragma unroll
        for (int iu = 0; iu < VU; ++iu) {
          const int u = lane + 64 * iu;
          if (VUN % 64 == 0 || u < VUN) {
            const int c = u % (D / 8), gg = u / (D / 8);
            const int v0 = rowb + 4 * gg * (D * 2) + 16 * c, v1 = v0 + 16 * (D * 2);
#pragma unroll
            for (int kk = 0; kk < 8; ++kk)
              raw.vr[iu][kk] =
                  __builtin_amdgcn_raw_buffer_load_b128(rv, (kk < 4 ? v0 : v1) + (kk & 3) * (D * 2), 0, ATTN_DEC_VNT ? 2 : 0);
          }
        }
      }
    };
#else
    auto load = [&](Raw &, int) {};   // (host pass: the kernel body is not built)
#endif
    auto compute = [&](const Raw &raw, int kb) {
      u32x4 kr[NKR];
      if constexpr (Q8) {
        // the scale rows through LDS; each lane then reads the scales it needs
  #pragma unroll
        for (int j = 0; j < Raw::SW; ++j)
          *reinterpret_cast<uint32_t *>(sct + lane * (D / 32) + 2 * j) = raw.sc[j];
        __syncthreads();
        // V: each 8-code unit dequantized straight into the block's LDS tile
        // (rows as loaded), so that no register copy of the whole block is live
  #pragma unroll
        for (int iu = 0; iu < VU; ++iu) {
          const int u = lane + 64 * iu;
          if (VUN % 64 == 0 || u < VUN) {
            const int c = u % (D / 8), gg = u / (D / 8);
  #pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
              const int row = kk < 4 ? 4 * gg + kk : 16 + 4 * gg + kk - 4;
              const uint16_t sv = sct[(32 + row) * (D / 32) + c / 4];
              st16(vt + row * VRS + 8 * c, dequant8(raw.vq[iu][kk][0], raw.vq[iu][kk][1], half_bits_to_float(sv)));
            }
          }
        }
  #pragma unroll
        for (int rb = 0; rb < 2; ++rb)
  #pragma unroll
          for (int ks = 0; ks < KST; ++ks) {
            // chunk ks = dims 64 (ks / 2) + 16 g + 8 (ks % 2): half of piece ks / 2,
            // in block 2 (ks / 2) + g / 2 of key row 16 rb + ql
            const int i = ks >> 1, h = ks & 1;
            const uint16_t sk = sct[(16 * rb + ql) * (D / 32) + 2 * i + (g >> 1)];
            kr[rb * KST + ks] = dequant8(raw.kq[rb][i][2 * h], raw.kq[rb][i][2 * h + 1], half_bits_to_float(sk));
          }
      } else {
  #pragma unroll
        for (int i = 0; i < NKR; ++i) kr[i] = raw.kr[i];
        // V block -> LDS, rows as loaded
  #pragma unroll
        for (int iu = 0; iu < VU; ++iu) {
          const int u = lane + 64 * iu;
          if (VUN % 64 == 0 || u < VUN) {
            const int c = u % (D / 8), gg = u / (D / 8);
  #pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
              const int row = kk < 4 ? 4 * gg + kk : 16 + 4 * gg + kk - 4;
              st16(vt + row * VRS + 8 * c, raw.vr[iu][kk]);
            }
          }
        }
      }
      // S^T = K Q^T: 32 keys x 16 queries per column block
      f32x4 s[NCB][2];
  #pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
  #pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          s[cb][rb] = f32x4{};
  #pragma unroll
          for (int ks = 0; ks < KST; ++ks)
            s[cb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[rb * KST + ks]), qf[cb][ks], s[cb][rb], 0, 0, 0);
        }
      __syncthreads();
      const bool partial = kb + 32 > kfull || kb < klo_all;
      bf16x8 pb[NCB];
  #pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        uint32_t vis = 0xffu;
        if (partial) {
          vis = 0;
  #pragma unroll
          for (int rb = 0; rb < 2; ++rb)
  #pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const int key = kb + 16 * rb + 4 * g + rr;
              const bool vv = key < k1 && key < kcol[cb] && key >= klo[cb];
              vis |= (vv ? 1u : 0u) << (4 * rb + rr);
              s[cb][rb][rr] = vv ? s[cb][rb][rr] : maskval;
            }
        }
        float red;
        if (cpos) {
          red = fmax3(s[cb][0][0], s[cb][0][1], s[cb][0][2]);
          red = fmax3(red, s[cb][0][3], s[cb][1][0]);
          red = fmax3(red, s[cb][1][1], s[cb][1][2]);
          red = __builtin_fmaxf(red, s[cb][1][3]);
          red = __builtin_fmaxf(red, xor16(red));
          red = __builtin_fmaxf(red, xor32(red));
        } else {
          red = fmin3(s[cb][0][0], s[cb][0][1], s[cb][0][2]);
          red = fmin3(red, s[cb][0][3], s[cb][1][0]);
          red = fmin3(red, s[cb][1][1], s[cb][1][2]);
          red = __builtin_fminf(red, s[cb][1][3]);
          red = __builtin_fminf(red, xor16(red));
          red = __builtin_fminf(red, xor32(red));
        }
        const float mt = red * cexp;
        const bool need = mt > m_run[cb] + ATTN_RESCALE_SLACK;
        if (wave_any(need)) {
          const float mnew = need ? mt : m_run[cb];
          const float alpha = need ? fast_exp2(m_run[cb] - mnew) : 1.f;
          l_run[cb] *= alpha;
  #pragma unroll
          for (int db = 0; db < D / 16; ++db) o[cb][db] *= alpha;
          m_run[cb] = mnew;
        }
        const float nm = -m_run[cb];
        float p[8];
  #pragma unroll
        for (int i = 0; i < 8; ++i) {
          float e = fast_exp2(__builtin_fmaf(s[cb][i >> 2][i & 3], cexp, nm));
          if (partial) e = ((vis >> i) & 1u) ? e : 0.f;
          p[i] = e;
        }
        l_run[cb] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
        pb[cb] = pack8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
      }
      // O^T += V^T P^T
  #pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        // V^T operand, lane (ql, g): dim 16 db + ql of key rows 4 g + 0..3 and
        // 16 + 4 g + 0..3 (the keys of this lane's P^T elements).  The 16
        // lanes of group g address rows 4 g + (ql >> 2), 4 dims from
        // 16 db + 4 (ql & 3); the transposing read hands each its own dim.
        const uint16_t *vp = vt + (4 * g + (ql >> 2)) * VRS + 16 * db + 4 * (ql & 3);
        const bf16x4 lo = lds_tr16(vp);
        const bf16x4 hi = lds_tr16(vp + 16 * VRS);
        const bf16x8 vop = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  #pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
          o[cb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pb[cb], o[cb][db], 0, 0, 0);
      }
      __syncthreads();
    };

    const int nblk = (k1 - k0 + 31) / 32;
    if constexpr (D <= 128 && NCB <= ATTN_DEC_DBUF_NCB) {
      // two register sets: block i+1 is in flight while block i is computed
      Raw rA, rB;
      load(rA, k0);
      for (int bi = 0; bi < nblk; bi += 2) {
        if (bi + 1 < nblk) load(rB, k0 + 32 * (bi + 1));
        compute(rA, k0 + 32 * bi);
        if (bi + 1 >= nblk) break;
        if (bi + 2 < nblk) load(rA, k0 + 32 * (bi + 2));
        compute(rB, k0 + 32 * (bi + 1));
      }
    } else {
      // D = 256, or four column blocks: one register set (a second would not
      // fit next to the accumulators)
      Raw rA;
      for (int bi = 0; bi < nblk; ++bi) {
        load(rA, k0 + 32 * bi);
        compute(rA, k0 + 32 * bi);
      }
    }

    // ---- this piece's result ---------------------------------------------
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      float lt = l_run[cb];
      lt += xor16(lt);
      lt += xor32(lt);
      // a row that sees no key of this piece (only with T > 1) has l = 0
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const int qi = 16 * cb + ql;
      if (qi < gcnt) {
        const size_t row = ((size_t)b * a.Hq + hkv * a.G) * a.T + gq0 + qi;
        const float lse_c = lt > 0.f ? m_run[cb] * ATTN_LN2 + __logf(lt) : -__builtin_inff();
        if (whole) {
#pragma unroll
          for (int db = 0; db < D / 16; ++db) {
            bf16x4 v4;
            v4[0] = (__bf16)(o[cb][db][0] * inv);
            v4[1] = (__bf16)(o[cb][db][1] * inv);
            v4[2] = (__bf16)(o[cb][db][2] * inv);
            v4[3] = (__bf16)(o[cb][db][3] * inv);
            *reinterpret_cast<bf16x4 *>(a.out + row * D + 16 * db + 4 * g) = v4;
          }
          if (a.lse != nullptr && g == 0) a.lse[row] = lse_c;
        } else {
          const size_t pr = (size_t)slot * GW + qi;
          float *po = a.part_o + pr * D;
#pragma unroll
          for (int db = 0; db < D / 16; ++db) *reinterpret_cast<f32x4 *>(po + 16 * db + 4 * g) = o[cb][db] * inv;
          if (g == 0) a.part_lse[pr] = lse_c;
        }
      }
    }

    // ---- next segment (skipping empty sequences) --------------------------
    r += take;
    if (r >= r1) break;
    blk = 0;
    if (++hh == HH) {
      hh = 0;
      do {
        ++b;
      } while (b < a.B && a.pre[b + 1] == a.pre[b]);
      if (b >= a.B) break;  // not reached: r < r1 <= total implies a later block
      nb = a.pre[b + 1] - a.pre[b];
    }
  }
}

// s_waitcnt vmcnt(n) (n < 64), other counters left alone
#define ATTN_DEC_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 15) | ((((n) >> 4) & 3) << 14))
// s_waitcnt lgkmcnt(0), other counters left alone
#define ATTN_DEC_WAIT_LDS() __builtin_amdgcn_s_waitcnt(0xC07F)
// cache policy of decode_wide_kernel's direct loads: 2 = nontemporal (nt),
// as for the streaming loads of decode_main_kernel: each K/V row is read once
#ifndef ATTN_DEC_WCPOL
#define ATTN_DEC_WCPOL 2
#endif

// Wide row groups (17 to 64 query rows of a KV head: G * T > 16): the same
// flat split, pieces and combine as decode_main_kernel, with the matrix work
// of the prefill kernel.  NC blocks of 32 query rows per wave; per 32-key
// block:
//  * K and V rows move HBM -> LDS with direct loads (no registers), two
//    blocks in flight, rows outside the piece's keys read from its edge (and
//    masked), K rows XOR-swizzled for the b128 operand reads, V rows for the
//    transposing reads;
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (32 keys x 32 rows; each K
//    operand read serves every row block), so a lane holds one query row and
//    16 keys: row max and sum are lane-local plus one v_permlane32_swap;
//  * O^T += V^T P^T with P^T packed from the accumulators and V^T read with
//    ds_read_b64_tr_b16.
template <int D, int NC>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(NC == 1 ? 2 : 1))) void decode_wide_kernel(DecodeArgs a) {
  constexpr int TILE = 32 * D;            // elements of one 32-key K or V tile
  constexpr int NBLK = TILE * 2 / 1024;   // 1 KiB direct loads per tile
  constexpr int RPB = 512 / D;            // rows per 1 KiB
  constexpr int CPR = D / 8;              // 16-byte chunks per row
  constexpr int NLD = 2 * NBLK;           // direct loads per 32-key block
  __shared__ __attribute__((aligned(1024))) uint16_t kb0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t kb1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t vb0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t vb1[TILE];

  const int lane = threadIdx.x;
  const int ql = lane & 31, hf = lane >> 5;
  const long long W = gridDim.x, w = blockIdx.x;
  const long long HH = (long long)a.Hkv * a.n_hg;
  const long long total = a.pre[a.B] * HH;
  const long long q = total / W, rem = total % W;
  long long r = q * w + min(w, rem);
  const long long r1 = r + q + (w < rem ? 1 : 0);
  if (r >= r1) return;
  int b;
  {
    int lo = 0, hi = a.B;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (HH * a.pre[mid] <= r) lo = mid;
      else hi = mid;
    }
    b = lo;
  }
  long long nb = a.pre[b + 1] - a.pre[b];
  long long off = r - HH * a.pre[b];
  int hseg = (int)(off / nb);
  long long blk = off - hseg * nb;

  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  const float cexp = a.c;
  const bool cpos = cexp >= 0.f;
  const float maskval = cpos ? -__builtin_inff() : __builtin_inff();
  const int GT = a.G * a.T;
  const int GW = min(GT, decode_group(D));

  // per-lane LDS offsets (elements) of the operands, as in the prefill
  // kernel: K row ql, chunk 2 ks + hf; V^T rows 4 hf + (j16 >> 2) of each
  // 16-key step
  const int g16 = lane >> 4, j16 = lane & 15;
  constexpr int NKO = D / 16 < 8 ? D / 16 : 8;
  constexpr int NVO = D / 32 < 4 ? D / 32 : 4;
  int koffs[NKO];
#pragma unroll
  for (int ks = 0; ks < NKO; ++ks) koffs[ks] = ql * D + 8 * ((2 * ks + hf) ^ kswz<D>(ql));
  int voffs[NVO];
  {
    const int vr = 4 * hf + (j16 >> 2);
    const int tv = vswz<D>(vr) >> 2;
    const int cin = 2 * (g16 & 1) + ((j16 & 3) >> 1);
#pragma unroll
    for (int db = 0; db < NVO; ++db) voffs[db] = vr * D + 8 * (4 * (db ^ tv) + cin) + 4 * (j16 & 1);
  }
  auto koff = [&](int ks) __attribute__((always_inline)) { return koffs[ks % NKO] + (ks / NKO) * 128; };
  auto voff = [&](int db) __attribute__((always_inline)) { return voffs[db % NVO] + (db / NVO) * 128; };

  while (r < r1) {
    const long long take = min(nb - blk, r1 - r);
    const int hkv = hseg / a.n_hg, hg = hseg - hkv * a.n_hg;
    const int gq0 = hg * decode_group(D);
    const int gcnt = min(decode_group(D), GT - gq0);
    const int n = max(0, min(a.lens[b], a.Lmax));
    const int kseg = seg_begin(a, n);
    const int kmin = a.window ? max(0, n - a.T - a.window + 1) : 0;
    const int k0 = kseg + (int)(blk * 32);
    const int k1 = min(n, kseg + (int)((blk + take) * 32));
    const bool whole = (blk == 0) && (take == nb);
    // this lane's query row in each row block and its visible keys
    // [klo, kcol): row t of the T new rows sees keys up to n - T + t
    int kcol[NC], klo[NC];
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) {
      kcol[cb] = n - a.T + 1 + (gq0 + 32 * cb + ql) % a.T;
      klo[cb] = a.window ? kcol[cb] - a.window : -0x7fffffff;
    }
    const int kfull = min(k1, n - a.T + 1);
    const int klo_all = a.window ? n - a.window : -0x7fffffff;
    const long long slot = (long long)b * HH + hseg + w;

    // Q^T operands: row 32 cb + ql, dims 16 ks + 8 hf ...
    bf16x8 qf[NC][D / 16];
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) {
      const int qi = 32 * cb + ql;
      const uint16_t *qp = a.q + (((size_t)b * a.Hq + hkv * a.G) * a.T + gq0 + min(qi, gcnt - 1)) * D + 8 * hf;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) qf[cb][ks] = as_bf16x8(qi < gcnt ? ld16(qp + 16 * ks) : zero4);
    }
    const size_t base = ((size_t)b * a.Hkv + hkv) * (size_t)a.Lmax * D;
    const uint16_t *kg = a.kc + base;
    const uint16_t *vg = a.vc + base;

    f32x16 o[NC][D / 32];
    float m_run[NC], l_run[NC];
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) {
      m_run[cb] = -__builtin_inff();
      l_run[cb] = 0.f;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[cb][db] = f32x16{};
    }

    // the 32-key block at kb into LDS (rows clamped into [kmin, k1): such
    // rows are masked)
    auto dma = [&](uint16_t *kd, uint16_t *vd, int kb) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < NBLK; ++i) {
        const int row = i * RPB + lane / CPR;
        const size_t key = (size_t)min(max(kb + row, kmin), k1 - 1);
        const int ck = (lane % CPR) ^ kswz<D>(row);
        const int cv = (lane % CPR) ^ vswz<D>(row);
        __builtin_amdgcn_global_load_lds((glb_void_t *)(kg + key * D + 8 * ck), (lds_void_t *)(kd + i * 512), 16, 0,
                                         ATTN_DEC_WCPOL);
        __builtin_amdgcn_global_load_lds((glb_void_t *)(vg + key * D + 8 * cv), (lds_void_t *)(vd + i * 512), 16, 0,
                                         ATTN_DEC_WCPOL);
      }
    };

    auto compute = [&](const uint16_t *kt, const uint16_t *vt, int kb) __attribute__((always_inline)) {
      // S^T = K Q^T, every K operand read serving the NC row blocks
      f32x16 s[NC];
#pragma unroll
      for (int cb = 0; cb < NC; ++cb) s[cb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 kop = as_bf16x8(ld16(kt + koff(ks)));
#pragma unroll
        for (int cb = 0; cb < NC; ++cb) s[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qf[cb][ks], s[cb], 0, 0, 0);
      }
      {
        constexpr int N = D / 16, A = N < 4 ? N : 4;
        __builtin_amdgcn_sched_group_barrier(0x100, A, 0);
#pragma unroll
        for (int i = 0; i < N - A; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, NC, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, NC * A, 0);
      }
      const bool partial = kb + 32 > kfull || kb < klo_all;
      bf16x8 pb[NC][2];
#pragma unroll
      for (int cb = 0; cb < NC; ++cb) {
        uint32_t vis = 0xffffu;
        if (partial) {
          vis = 0;
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            const int key = kb + 8 * (rr >> 2) + 4 * hf + (rr & 3);
            const bool vv = key < k1 && key < kcol[cb] && key >= klo[cb];
            vis |= (vv ? 1u : 0u) << rr;
            s[cb][rr] = vv ? s[cb][rr] : maskval;
          }
        }
        float red;
        if (cpos) {
          red = fmax3(s[cb][0], s[cb][1], s[cb][2]);
#pragma unroll
          for (int i = 3; i < 15; i += 2) red = fmax3(red, s[cb][i], s[cb][i + 1]);
          red = pair_max(__builtin_fmaxf(red, s[cb][15]));
        } else {
          red = fmin3(s[cb][0], s[cb][1], s[cb][2]);
#pragma unroll
          for (int i = 3; i < 15; i += 2) red = fmin3(red, s[cb][i], s[cb][i + 1]);
          red = pair_min(__builtin_fminf(red, s[cb][15]));
        }
        const float mt = red * cexp;
        const bool need = mt > m_run[cb] + ATTN_RESCALE_SLACK;
        if (wave_any(need)) {
          const float mnew = need ? mt : m_run[cb];
          const float alpha = need ? fast_exp2(m_run[cb] - mnew) : 1.f;
          l_run[cb] *= alpha;
#pragma unroll
          for (int db = 0; db < D / 32; ++db) o[cb][db] *= alpha;
          m_run[cb] = mnew;
        }
        const float nm = -m_run[cb];
        float p[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float e = fast_exp2(__builtin_fmaf(s[cb][i], cexp, nm));
          // a hidden score is +-inf; with c == 0 the product would be NaN
          if (partial) e = ((vis >> i) & 1u) ? e : 0.f;
          p[i] = e;
        }
        float t8[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) t8[i] = p[i] + p[i + 8];
        l_run[cb] += ((t8[0] + t8[1]) + (t8[2] + t8[3])) + ((t8[4] + t8[5]) + (t8[6] + t8[7]));
        pb[cb][0] = pack8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
        pb[cb][1] = pack8(p[8], p[9], p[10], p[11], p[12], p[13], p[14], p[15]);
      }
      // O^T += V^T P^T, every V^T operand read serving the NC row blocks
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int kq = 0; kq < 2; ++kq) {
          const uint16_t *vp = vt + 16 * kq * D + voff(db);
          const bf16x4 lo = lds_tr16(vp);
          const bf16x4 hi = lds_tr16(vp + 8 * D);
          const bf16x8 vop = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
          for (int cb = 0; cb < NC; ++cb)
            o[cb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb[cb][kq], o[cb][db], 0, 0, 0);
        }
      }
      {
        constexpr int N = 2 * (D / 32), A = N < 3 ? N : 3;
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * A, 0);
#pragma unroll
        for (int i = 0; i < N - A; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, NC, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, NC * A, 0);
      }
    };

    // two blocks in flight: block i in (kb[i % 2], vb[i % 2]); the loads of
    // block i + 2 go into the buffers of block i once its reads are done
    const int nblk = (k1 - k0 + 31) / 32;
    auto step = [&](int bi, uint16_t *kt, uint16_t *vt) __attribute__((always_inline)) {
      if (bi + 1 < nblk) ATTN_DEC_WAIT_VM(NLD);
      else ATTN_DEC_WAIT_VM(0);
      compute(kt, vt, k0 + 32 * bi);
      if (bi + 2 < nblk) {
        ATTN_DEC_WAIT_LDS();
        dma(kt, vt, k0 + 32 * (bi + 2));
      }
    };
    ATTN_DEC_WAIT_LDS();   // the previous piece's reads of these buffers are done
    dma(kb0, vb0, k0);
    if (nblk > 1) dma(kb1, vb1, k0 + 32);
    for (int bi = 0; bi < nblk; bi += 2) {
      step(bi, kb0, vb0);
      if (bi + 1 >= nblk) break;
      step(bi + 1, kb1, vb1);
    }

    // ---- this piece's result: lane (row 32 cb + ql) holds dims
    // 32 db + 8 j + 4 hf + (0..3) -----------------------------------------
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) {
      const float lt = pair_sum(l_run[cb]);
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const int qi = 32 * cb + ql;
      if (qi < gcnt) {
        const size_t row = ((size_t)b * a.Hq + hkv * a.G) * a.T + gq0 + qi;
        const float lse_c = lt > 0.f ? m_run[cb] * ATTN_LN2 + __logf(lt) : -__builtin_inff();
        if (whole) {
#pragma unroll
          for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              bf16x4 v4;
#pragma unroll
              for (int i = 0; i < 4; ++i) v4[i] = (__bf16)(o[cb][db][4 * j + i] * inv);
              *reinterpret_cast<bf16x4 *>(a.out + row * D + 32 * db + 8 * j + 4 * hf) = v4;
            }
          if (a.lse != nullptr && hf == 0) a.lse[row] = lse_c;
        } else {
          const size_t pr = (size_t)slot * GW + qi;
          float *po = a.part_o + pr * D;
#pragma unroll
          for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const f32x4 v4 = {o[cb][db][4 * j] * inv, o[cb][db][4 * j + 1] * inv, o[cb][db][4 * j + 2] * inv,
                                o[cb][db][4 * j + 3] * inv};
              *reinterpret_cast<f32x4 *>(po + 32 * db + 8 * j + 4 * hf) = v4;
            }
          if (hf == 0) a.part_lse[pr] = lse_c;
        }
      }
    }

    // ---- next segment (skipping empty sequences) --------------------------
    r += take;
    if (r >= r1) break;
    blk = 0;
    if (++hseg == HH) {
      hseg = 0;
      do {
        ++b;
      } while (b < a.B && a.pre[b + 1] == a.pre[b]);
      if (b >= a.B) break;
      nb = a.pre[b + 1] - a.pre[b];
    }
  }
}

// Merge the pieces of every (sequence, query head) whose segment was split
// between waves; also writes out = 0 / lse = -inf for empty sequences.  One
// wave per row: piece lse values are read one per lane (64 per round) and
// reduced across the wave; each lane accumulates D/64 output elements.
template <int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(DecodeArgs a, int W) {
  const int row = blockIdx.x;  // (b * Hq + h) * T + t
  const int HT = a.Hq * a.T, GT = a.G * a.T;
  const int b = row / HT, ht = row - b * HT;
  const int lane = threadIdx.x;
  const int hkv = ht / GT, gfull = ht - hkv * GT;   // row within the KV head's G * T rows
  const int hg = gfull / decode_group(D), qi = gfull - hg * decode_group(D);
  const long long HH = (long long)a.Hkv * a.n_hg;
  const long long hh = (long long)hkv * a.n_hg + hg;
  const long long nb = a.pre[b + 1] - a.pre[b];
  uint16_t *op = a.out + (size_t)row * D;
  if (nb == 0) {
    for (int d = lane; d < D; d += 64) op[d] = 0;
    if (a.lse != nullptr && lane == 0) a.lse[row] = -__builtin_inff();
    return;
  }
  const long long total = a.pre[a.B] * HH;
  const long long s0 = HH * a.pre[b] + hh * nb;       // first flat block of the segment
  const long long w0 = wave_of(s0, total, W), w1 = wave_of(s0 + nb - 1, total, W);
  if (w0 == w1) return;  // one wave covered it and wrote the result
  const int GW = min(GT, decode_group(D));
  const long long seg = (long long)b * HH + hh;
  const int np = (int)(w1 - w0 + 1);
  auto prow = [&](int c) { return ((size_t)(seg + w0 + c) * GW + qi); };
  float M = -__builtin_inff();
  float x0 = -__builtin_inff();   // this lane's piece lse among the first 64, kept
  for (int c0 = 0; c0 < np; c0 += 64) {
    const float x = (c0 + lane < np) ? a.part_lse[prow(c0 + lane)] : -__builtin_inff();
    if (c0 == 0) x0 = x;
    M = __builtin_fmaxf(M, x);
  }
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) M = __builtin_fmaxf(M, __shfl_xor(M, sh));
  if (M == -__builtin_inff()) {  // the row saw no key in any piece (only with T > 1)
    for (int d = lane; d < D; d += 64) op[d] = 0;
    if (a.lse != nullptr && lane == 0) a.lse[row] = -__builtin_inff();
    return;
  }
  float Z = 0.f;
  float acc[D / 64];
#pragma unroll
  for (int i = 0; i < D / 64; ++i) acc[i] = 0.f;
  for (int c0 = 0; c0 < np; c0 += 64) {
    const float x = c0 == 0 ? x0 : ((c0 + lane < np) ? a.part_lse[prow(c0 + lane)] : -__builtin_inff());
    const float wl = (c0 + lane < np) ? __expf(x - M) : 0.f;
    Z += wl;
    const int cn = min(64, np - c0);
    int c = 0;
    // four pieces' loads issued together, then added in piece order
    for (; c + 4 <= cn; c += 4) {
      float pv[4][D / 64];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float *po = a.part_o + prow(c0 + c + u) * D;
#pragma unroll
        for (int i = 0; i < D / 64; ++i) pv[u][i] = po[lane + 64 * i];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float wgt = __shfl(wl, c + u);
#pragma unroll
        for (int i = 0; i < D / 64; ++i) acc[i] = __builtin_fmaf(wgt, pv[u][i], acc[i]);
      }
    }
    for (; c < cn; ++c) {
      const float wgt = __shfl(wl, c);
      const float *po = a.part_o + prow(c0 + c) * D;
#pragma unroll
      for (int i = 0; i < D / 64; ++i) acc[i] = __builtin_fmaf(wgt, po[lane + 64 * i], acc[i]);
    }
  }
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) Z += __shfl_xor(Z, sh);
  const float inv = 1.f / Z;
#pragma unroll
  for (int i = 0; i < D / 64; ++i) {
    const __bf16 hv = (__bf16)(acc[i] * inv);
    op[lane + 64 * i] = __builtin_bit_cast(uint16_t, hv);
  }
  if (a.lse != nullptr && lane == 0) a.lse[row] = M + __logf(Z);
}

template <int D, int NCB>
static hipError_t launch_t(const DecodeArgs &a, int W, hipStream_t s) {
  hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(1024), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.kscale != nullptr) hipLaunchKernelGGL((decode_main_kernel<D, NCB, true>), dim3(W), dim3(64), 0, s, a);
  else hipLaunchKernelGGL((decode_main_kernel<D, NCB, false>), dim3(W), dim3(64), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(a.B * a.Hq * a.T), dim3(64), 0, s, a, W);
  return hipGetLastError();
}

template <int D, int NC>
static hipError_t launch_w(const DecodeArgs &a, int W, hipStream_t s) {
  hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(1024), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_wide_kernel<D, NC>), dim3(W), dim3(64), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(a.B * a.Hq * a.T), dim3(64), 0, s, a, W);
  return hipGetLastError();
}

template <int D>
constexpr bool kDecodeWide = D <= 128 && (ATTN_DEC_WIDE & (D == 64 ? 1 : 2)) != 0;

template <int D>
static hipError_t launch_d(const DecodeArgs &a, int W, hipStream_t s) {
  const int gt = a.G * a.T;
  const int gw = gt < decode_group(D) ? gt : decode_group(D);
  const int ncb = (gw + 15) / 16;
  if constexpr (D <= 128) {
    if (a.wide) return launch_w<D, 2>(a, W, s);
  }
  if (ncb == 1) return launch_t<D, 1>(a, W, s);
  if (ncb == 2 || D == 256) return launch_t<D, 2>(a, W, s);   // (D = 256: groups of at most 32 rows)
  return launch_t<D, D == 256 ? 2 : 4>(a, W, s);
}

hipError_t launch_decode(const DecodeArgs &a, int D, int W, hipStream_t s) {
  switch (D) {
    case 64: return launch_d<64>(a, W, s);
    case 128: return launch_d<128>(a, W, s);
    case 256: return launch_d<256>(a, W, s);
    default: return hipErrorInvalidValue;
  }
}

// Resident 64-thread workgroups of the main kernel per CU for GW query rows
// per wave group (q8: the int8-cache kernel).
bool decode_use_wide(int D, int GW, bool q8, long long blocks) {
  const int gw = GW < decode_group(D) ? GW : decode_group(D);
  const bool built = D == 64 ? kDecodeWide<64> : D == 128 ? kDecodeWide<128> : kDecodeWide<256>;
  return built && !q8 && gw > 32 && blocks >= kDecodeWideMinBlocks;
}

hipError_t decode_waves_per_cu(int D, int GW, bool q8, bool wide, int *out) {
  const int gw = GW < decode_group(D) ? GW : decode_group(D);
  const int ncb = (gw + 15) / 16;
  const void *f = nullptr;
  if (wide) {
    if (D == 64) f = (const void *)&decode_wide_kernel<64, 2>;
    else if (D == 128) f = (const void *)&decode_wide_kernel<128, 2>;
    else return hipErrorInvalidValue;   // not built for D = 256 (its registers spill)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(out, f, 64, 0);
  }
#define ATTN_PICK(DD, NN)                                                                \
  f = q8 ? reinterpret_cast<const void *>(&decode_main_kernel<DD, NN, true>)           \
         : reinterpret_cast<const void *>(&decode_main_kernel<DD, NN, false>)
  if (D == 64) { if (ncb == 1) ATTN_PICK(64, 1); else if (ncb == 2) ATTN_PICK(64, 2); else ATTN_PICK(64, 4); }
  else if (D == 128) { if (ncb == 1) ATTN_PICK(128, 1); else if (ncb == 2) ATTN_PICK(128, 2); else ATTN_PICK(128, 4); }
  else { if (ncb == 1) ATTN_PICK(256, 1); else ATTN_PICK(256, 2); }
#undef ATTN_PICK
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(out, f, 64, 0);
}

}  // namespace attn
