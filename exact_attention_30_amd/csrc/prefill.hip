// Prefill: exact GQA attention of Lq query rows over Lk keys, causal mask
// anchored bottom-right, computed tile by tile with an online softmax.
//
// Method (pages, by title): "어텐션 구현 고르기, SDPA·FlashAttention 메모리와
// GPU 비용", section "eager 어텐션 메모리, 길이에 따라 얼마나 커지나" (split the
// score table into blocks held on chip, keep a per-row maximum and sum, no
// approximation) and section "긴 입력에서 어텐션 연산이 차지하는 비중" (blocks
// the causal mask hides entirely are skipped); section "is_causal 마스크 정렬…"
// for the bottom-right alignment; "Как NVIDIA учит нейросети думать
// быстрее…", section on group size (G query heads read one KV head).
//
// gfx950 design
//  * A workgroup of 8 wave64s (D = 256: 4, one per SIMD, for registers) covers
//    32 query rows per wave of up to 8 query heads that share one KV head;
//    every K/V tile it stages in LDS serves all of them.
//  * Each wave computes the transposed score block S^T = K Q^T with
//    v_mfma_f32_32x32x16_bf16 (keys on the M side, queries on the N side, Q in
//    registers).  In the accumulator layout a lane holds one query column and
//    16 keys per 32-key block, so the row max and row sum are lane-local plus
//    one v_permlane32_swap between the two wave halves.
//  * P^T (bf16, round to nearest even) feeds O^T += V^T P^T straight from
//    those registers.  V stays row-major in LDS; its V^T operand is read with
//    ds_read_b64_tr_b16 (a 4 x 16 transpose per 16-lane group), two reads per
//    MFMA, in the key order the P^T registers hold.
//  * Tiles move HBM -> LDS with buffer_load_dwordx4 ... lds (no registers, no
//    ds_write): a buffer resource per tile (scalar base and size, so rows
//    past the keys read as zeros) and a fixed offset per lane, so a load
//    costs no vector instruction.  Rows are unpadded; a row's 16-byte chunks
//    are XOR-swizzled so that the b128 K reads and the transposing V reads
//    are free of bank conflicts.  K and V are double-buffered in four
//    separate LDS arrays.
//  * Softmax in the log2 domain: p = exp2(s*c - m) with c = scale*log2(e).
//    The running maximum only has to keep the exponentials from overflowing
//    the fp32 sums: prefill_kernel exponentiates a tile against it first and
//    takes the tile's maximum (and rescales O and l) only when some sum
//    exceeds 2^32; prefill_iw_kernel raises it only past a slack of 2^8.
//    The row sum adds the fp32 exponentials (before their rounding to
//    bf16), so that the log-sum-exp is that of the true normaliser.
//  * Two schedules.  prefill_kernel pairs the waves of a SIMD in two groups
//    that alternate matrix work and softmax (one group's exponentials run
//    beside the other group's MFMAs).  prefill_iw_kernel runs one schedule in
//    every wave and interleaves each wave's own exponentials and row sums
//    with its own MFMAs (sched_group_barrier); it is the faster one for
//    D = 64 and for D = 256 (one wave per SIMD), the ping-pong for D = 128.
//  * Causal: tiles past the workgroup's last visible key are skipped, the
//    mask is evaluated only on tiles that cross the diagonal, the end of the
//    keys or a window's lower edge.  Workgroups are issued heaviest first, and
//    consecutive workgroup ids are spread over the 8 XCDs so that each XCD
//    works on one KV head at a time (its K/V stay in that XCD's L2).
//  * Small grids split each query block's keys over several workgroups and
//    merge the partial results with their log-sum-exps (combine kernel).
#include <type_traits>

#include "common.h"
#include "kernels.h"

// Scheduling choices (compile-time):
//  ATTN_PF_PV_AHEAD     V^T operand reads issued this many MFMAs ahead
//  ATTN_PF_QK_AHEAD     K operand reads issued this many MFMAs ahead
#ifndef ATTN_PF_PV_AHEAD
#define ATTN_PF_PV_AHEAD 2
#endif
#ifndef ATTN_PF_QK_AHEAD
#define ATTN_PF_QK_AHEAD 2
#endif
//  ATTN_PF_IW           head dims that use prefill_iw_kernel (in-wave pipelined)
//                       rather than the two-group ping-pong prefill_kernel, as a
//                       bit mask: 1 = D 64, 2 = D 128, 4 = D 256
//  ATTN_PF_IW_V1/V2     vector instructions placed after each MFMA of bracket 1 / 2
#ifndef ATTN_PF_IW
#define ATTN_PF_IW 5
#endif
//  ATTN_PF_IW_QKA256 / ATTN_PF_IW_PVA256 / ATTN_PF_IW_V1_256   the read-ahead distances
//                       and bracket-1 vector instructions per MFMA of prefill_iw_kernel at D = 256
//                       (its registers leave room for reads further ahead)
#ifndef ATTN_PF_IW_QKA256
#define ATTN_PF_IW_QKA256 8
#endif
#ifndef ATTN_PF_IW_PVA256
#define ATTN_PF_IW_PVA256 5
#endif
#ifndef ATTN_PF_IW_V1_256
#define ATTN_PF_IW_V1_256 3
#endif
//  ATTN_PF_IW_SPREAD    head dims (bit mask as above) for which prefill_iw_kernel
//                       spreads its direct loads over the MFMAs
#ifndef ATTN_PF_IW_SPREAD
#define ATTN_PF_IW_SPREAD 4
#endif
#ifndef ATTN_PF_IW_V1
#define ATTN_PF_IW_V1 5
#endif
#ifndef ATTN_PF_IW_V2
#define ATTN_PF_IW_V2 2
#endif
//  ATTN_PF_LAZYMAX      prefill_kernel takes a tile's maximum only when its
//                       exponentials against the running max would exceed 2^32
//  ATTN_PF_IW_LAZY      prefill_iw_kernel likewise for D < 256 (its row sums then
//                       move into bracket 1, ahead of the P.V products that need
//                       the check)
#ifndef ATTN_PF_IW_LAZY
#define ATTN_PF_IW_LAZY 1
#endif
#ifndef ATTN_PF_LAZYMAX
#define ATTN_PF_LAZYMAX 1
#endif
//  ATTN_PF_PERSIST      head dims (bit mask as for ATTN_PF_IW) whose prefill runs
//                       as one resident workgroup per slot, each taking several
//                       work items, when the grid would fill two or more rounds
//                       of the device
#ifndef ATTN_PF_PERSIST
#define ATTN_PF_PERSIST 3
#endif
//  ATTN_PF_PIPE         prefill_kernel issues its MFMA operand reads ahead in
//                       explicit program order held by scheduling fences
#ifndef ATTN_PF_PIPE
#define ATTN_PF_PIPE 1
#endif
//  ATTN_PF_PRIO         wave priority in prefill_kernel's phases: 1 = the matrix
//                       phase raised, 2 = the softmax phase raised, 0 = neither
#ifndef ATTN_PF_PRIO
#define ATTN_PF_PRIO 1
#endif
//  ATTN_PF_ALT          prefill_kernel alternates the accumulators of consecutive
//                       MFMAs (key blocks of S^T, value blocks of O^T); the
//                       products into each accumulator keep their order
#ifndef ATTN_PF_ALT
#define ATTN_PF_ALT 1
#endif
#ifndef ATTN_PF_IW_ALT
#define ATTN_PF_IW_ALT 1
#endif
//  ATTN_PF_BK128        key-tile size for D = 128
#ifndef ATTN_PF_BK128
#define ATTN_PF_BK128 64
#endif

namespace attn {

//  ATTN_PF_NW256         waves per workgroup for D = 256 (8: two per SIMD; 4: one
//                       per SIMD, which leaves room for its O accumulators and Q
//                       operands without spilling)
#ifndef ATTN_PF_NW256
#define ATTN_PF_NW256 4
#endif
//  ATTN_PF_BK256        key-tile size for D = 256
#ifndef ATTN_PF_BK256
#define ATTN_PF_BK256 64
#endif

// whether head dim D runs on resident workgroups (ATTN_PF_PERSIST); the
// one-item form of prefill_iw_kernel is kept straight-line for the others
// (at D = 256 the item loop costs registers: 29 SGPRs spilled, -30%)
template <int D>
constexpr bool kPersist = (ATTN_PF_PERSIST & (D == 64 ? 1 : D == 128 ? 2 : 4)) != 0;
// prefill_kernel's MFMA order: consecutive MFMAs into different accumulators
constexpr bool kPfAlt = ATTN_PF_ALT != 0;
// the same for prefill_iw_kernel
constexpr bool kIwAlt = ATTN_PF_IW_ALT != 0;
constexpr int kPrioGemm = ATTN_PF_PRIO == 1 ? 1 : 0;
constexpr int kPrioSoft = ATTN_PF_PRIO == 2 ? 1 : 0;

template <int D>
constexpr int kPfThreads = (D == 256 ? ATTN_PF_NW256 : 8) * 64;


template <int D, int BK>
struct PrefillCfg {
  static constexpr int NW = kPfThreads<D> / 64;
  static constexpr int NT = NW * 64;
  static constexpr int CPR = D / 8;                   // 16-byte chunks per K/V row
  static constexpr int RPD = 512 / D;                 // rows per 1 KiB direct-to-LDS load
  static constexpr int TILE = BK * D;                 // elements per K or V tile
  static constexpr int DPW = TILE * 2 / 1024 / NW;    // (direct loads per tile and tensor) / waves
  static_assert(DPW * NW * 1024 == TILE * 2, "tile must split evenly over the waves");
  static_assert(BK % 32 == 0 && D % 32 == 0, "tile shape");
};


// s_waitcnt vmcnt(0), other counters left alone (expcnt 7, lgkmcnt 15)
#define ATTN_WAIT_VMEM() __builtin_amdgcn_s_waitcnt(0x0F70)

template <int D, int BK>
__global__ __launch_bounds__(kPfThreads<D>) void prefill_kernel(PrefillArgs a) {
  using C = PrefillCfg<D, BK>;
  // four separate arrays, so that reads of one buffer never wait for the
  // direct loads still filling another
  __shared__ __attribute__((aligned(1024))) uint16_t kb0[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t kb1[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t vb0[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t vb1[C::TILE];

  // ---- which tile: XCD-grouped, heaviest q-block first -------------------
  // One work item per workgroup, or (a.persist > 0) a.persist resident
  // workgroups that each take several: workgroup p runs on XCD p % 8 and
  // takes that XCD's items (the same XCD-grouped, heaviest-first order) in
  // rounds of a.persist / 8, alternately in increasing and decreasing order,
  // so that the sizes of its items add up to about the same total in every
  // workgroup.  The items left over by the grouping go one each to the first
  // workgroups.
  const int tf = a.total & ~7;
  const int per_x = tf >> 3, q8 = a.persist >> 3;
  const int px = blockIdx.x & 7, pi = blockIdx.x >> 3;
  bool tail_done = false;
  for (int it = 0;; ++it) {
  int t;
  if (a.persist == 0) {
    if (it > 0) break;
    const int bid = blockIdx.x;
    t = bid;
    if (bid < tf) t = (bid & 7) * per_x + (bid >> 3);
  } else {
    const int kx = it * q8 + ((it & 1) ? q8 - 1 - pi : pi);
    if (kx < per_x) {
      t = px * per_x + kx;
    } else if (!tail_done && (int)blockIdx.x < a.total - tf) {
      t = tf + blockIdx.x;
      tail_done = true;
    } else {
      break;
    }
  }
  const int sp = t % a.nsplit;  // key range of this workgroup
  t /= a.nsplit;
  int unit = t / a.n_qblk;
  const int r = t - unit * a.n_qblk;
  const int qblk = a.causal ? (a.n_qblk - 1 - r) : r;
  const int hg = unit % a.n_hg;
  unit /= a.n_hg;
  const int hkv = unit % a.Hkv;
  const int b = unit / a.Hkv;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int ql = lane & 31, hh = lane >> 5;
  const int head = hkv * a.G + hg * a.hpw + w / a.wph;
  const int q0w = qblk * a.Bq + (w % a.wph) * 32;
  const int qrow = q0w + ql;
  const int off = a.Lk - a.Lq;

  // keys this workgroup / this wave must visit
  const int qlast_wg = min(qblk * a.Bq + a.Bq, a.Lq) - 1;
  const int kend_wg = a.causal ? min(a.Lk, qlast_wg + off + 1) : a.Lk;
  int kend_w = 0;
  if (q0w < a.Lq) kend_w = a.causal ? min(a.Lk, min(q0w + 31, a.Lq - 1) + off + 1) : a.Lk;
  const int kmask_from = a.causal ? min(a.Lk, q0w + off + 1) : a.Lk;  // first key some row of the wave hides
  // sliding window: row i sees keys [i + off - window + 1, i + off]
  const int win = a.window;
  const int kbeg_wg = win ? max(0, qblk * a.Bq + off - win + 1) : 0;   // first key of the first row
  const int kbeg_w = win ? max(0, q0w + off - win + 1) : 0;             // ... of this wave's first row
  const int klo_until = win ? q0w + 31 + off - win + 1 : 0;             // keys below: hidden from some row
  const int qlo = win ? qrow + off - win + 1 : -0x7fffffff;             // this lane's first visible key
  // this workgroup's share of the tiles: [j0, j0 + nt)
  const int jbeg = kbeg_wg / BK;
  const int nt_all = (kend_wg + BK - 1) / BK - jbeg;
  const int j0 = jbeg + (int)((long long)nt_all * sp / a.nsplit);
  const int nt = jbeg + (int)((long long)nt_all * (sp + 1) / a.nsplit) - j0;

  // ---- Q (B operand of S^T), kept in registers ----------------------------
  const int qr = min(qrow, a.Lq - 1);
  const uint16_t *qp = a.q + (((size_t)b * a.Hq + head) * a.Lq + qr) * D;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) qf[ks] = as_bf16x8(ld16(qp + 16 * ks + 8 * hh));

  const size_t kvoff = ((size_t)b * a.Hkv + hkv) * (size_t)a.Lk * D;
  const uint16_t *kg = a.k + kvoff;
  const uint16_t *vg = a.v + kvoff;

  // Tile j of K or V straight from global memory into LDS, moved by the four
  // waves of one group: each wave moves 2 DPW blocks of 1 KiB; lane i fills
  // bytes [16 i, 16 i + 16) of a block, so it fetches the logical chunk that
  // the swizzle puts there.  Rows past the end of the keys are read from the
  // last row instead (the loads stay unconditional): such keys are masked,
  // so their K only meets -inf scores and their V only zero weights.
#if ATTN_DEVICE_PASS
  // a buffer resource over the rows of tile j that exist: the rows past the
  // end of the keys read as zeros (they are masked); the tile base is scalar
  // and a lane's offset fixed, so a load takes no vector work
  auto tile_rs = [&](const uint16_t *g, int j) __attribute__((always_inline)) {
    return buf_rsrc_uniform(g + (size_t)j * BK * D, (uint32_t)min(BK, a.Lk - j * BK) * (D * 2));
  };
  // the i-th of this wave's 2 DPW block loads of a tile
  auto dma_one = [&](auto rs, uint16_t *dst, int i, auto is_v) __attribute__((always_inline)) {
    constexpr bool V = decltype(is_v)::value;
    const int blk = (wu % (C::NW / 2)) * 2 * C::DPW + i;
    const int row = blk * C::RPD + lane / C::CPR;
    const int c = (lane % C::CPR) ^ (V ? vswz<D>(row) : kswz<D>(row));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t *)(dst + blk * 512), 16,
                                             (lane / C::CPR) * (D * 2) + 16 * c, blk * 1024, 0, 0);
  };
#endif
  auto dma = [&](const uint16_t *g, uint16_t *dst, int j, auto is_v) __attribute__((always_inline)) {
#if ATTN_DEVICE_PASS
    const auto rs = tile_rs(g, j);
#pragma unroll
    for (int i = 0; i < 2 * C::DPW; ++i) dma_one(rs, dst, i, is_v);
#endif
  };

  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = f32x16{};
  float m_run = -__builtin_inff();
  float l_run = 0.f;
  const float cexp = a.c;
  const bool cpos = cexp >= 0.f;
  const float maskval = cpos ? -__builtin_inff() : __builtin_inff();

  // per-lane LDS offsets (elements) of the MFMA operands.  K: row ql of the
  // 32-key block, logical chunk 2 ks + hh (+ 32 rb rows).  V^T: row
  // 4 hh + (j16 >> 2) of the 16-key block (+ 16 kb rows, + 8 for the upper
  // half), 4 columns starting at 32 db + 16 (g16 & 1) + 4 (j16 & 3).
  // The swizzles touch only the low 4 bits of a chunk index (K) or the low 2
  // bits of a 64-byte group index (V), so offsets repeat every 16 chunks / 4
  // groups up to a constant: only the first 8 K and 4 V offsets are kept.
  const int g16 = lane >> 4, j16 = lane & 15;
  constexpr int NKO = D / 16 < 8 ? D / 16 : 8;
  constexpr int NVO = D / 32 < 4 ? D / 32 : 4;
  int koffs[NKO];
#pragma unroll
  for (int ks = 0; ks < NKO; ++ks) koffs[ks] = ql * D + 8 * ((2 * ks + hh) ^ kswz<D>(ql));
  int voffs[NVO];
  {
    const int vr = 4 * hh + (j16 >> 2);
    const int tv = vswz<D>(vr) >> 2;
    const int cin = 2 * (g16 & 1) + ((j16 & 3) >> 1);
#pragma unroll
    for (int db = 0; db < NVO; ++db) voffs[db] = vr * D + 8 * (4 * (db ^ tv) + cin) + 4 * (j16 & 1);
  }
  auto koff = [&](int ks) __attribute__((always_inline)) { return koffs[ks % NKO] + (ks / NKO) * 128; };
  auto voff = [&](int db) __attribute__((always_inline)) { return voffs[db % NVO] + (db / NVO) * 128; };

  bf16x8 pb[BK / 16];
  // O^T += V^T P^T for one tile; the V^T operand comes from row-major V by
  // transposing reads
  auto pv = [&](const uint16_t *vs_) __attribute__((always_inline)) {
    constexpr int N = (D / 32) * (BK / 16);
    constexpr int A = ATTN_PF_PV_AHEAD;
    auto vread = [&](int i) __attribute__((always_inline)) {
      const int db = kPfAlt ? i % (D / 32) : i / (BK / 16), kb = kPfAlt ? i / (D / 32) : i % (BK / 16);
      const uint16_t *vp = vs_ + 16 * kb * D + voff(db);
      const bf16x4 lo = lds_tr16(vp);
      const bf16x4 hi = lds_tr16(vp + 8 * D);
      return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    if (ATTN_PF_PIPE) {
      // operand reads A MFMAs ahead, in a ring of A + 1 register sets; the
      // scheduling fences keep this order (left to itself the scheduler
      // moved every read next to its MFMA, which then waited for it)
      bf16x8 vr[A + 1];
#pragma unroll
      for (int i = 0; i < A && i < N; ++i) vr[i] = vread(i);
#pragma unroll
      for (int i = 0; i < N; ++i) {
        if (i + A < N) vr[(i + A) % (A + 1)] = vread(i + A);
        __builtin_amdgcn_sched_barrier(0);
        const int db = kPfAlt ? i % (D / 32) : i / (BK / 16), kb = kPfAlt ? i / (D / 32) : i % (BK / 16);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[i % (A + 1)], pb[kb], o[db], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int db = kPfAlt ? i % (D / 32) : i / (BK / 16), kb = kPfAlt ? i / (D / 32) : i % (BK / 16);
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vread(i), pb[kb], o[db], 0, 0, 0);
    }
    // keep the transposing reads ATTN_PF_PV_AHEAD MFMAs ahead of their use
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * A, 0);
#pragma unroll
    for (int i = 0; i < N - A; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, A, 0);
  };

  // Online-softmax update for one tile of S^T (this lane: one query, BK/2
  // keys): P = exp2(s*c - m) into pb, row sum into l_run, the running max
  // raised when needed.  MASKED: the tile crosses the diagonal or the end of
  // the keys and hidden scores hold maskval.
  //
  // The tile maximum is only needed when the exponentials would grow too
  // large for the fp32 sums (the running max only has to bound them), so the
  // tile is first exponentiated against the current running max; only if
  // some lane's tile sum exceeds 2^32 (or is not finite: the first tile,
  // where the running max is -inf) is the tile maximum taken, the running
  // max raised, O and l rescaled, and the tile exponentiated again.  The
  // running max therefore stays an actual maximum of scores seen (never above
  // the true one), and every exponential stays below 2^32.
  auto raise_max = [&](const f32x16(&s)[BK / 32]) __attribute__((always_inline)) {
    float red;
    if (cpos) {
      float mx[BK / 32][4];
#pragma unroll
      for (int rb = 0; rb < BK / 32; ++rb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          mx[rb][g] = fmax3(s[rb][4 * g], s[rb][4 * g + 1], __builtin_fmaxf(s[rb][4 * g + 2], s[rb][4 * g + 3]));
      red = mx[0][0];
#pragma unroll
      for (int rb = 0; rb < BK / 32; ++rb)
#pragma unroll
        for (int g = (rb == 0 ? 1 : 0); g < 4; g += 2)
          red = (g + 1 < 4) ? fmax3(red, mx[rb][g], mx[rb][g + 1]) : __builtin_fmaxf(red, mx[rb][g]);
      red = pair_max(red);
    } else {
      float mn[BK / 32][4];
#pragma unroll
      for (int rb = 0; rb < BK / 32; ++rb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          mn[rb][g] = fmin3(s[rb][4 * g], s[rb][4 * g + 1], __builtin_fminf(s[rb][4 * g + 2], s[rb][4 * g + 3]));
      red = mn[0][0];
#pragma unroll
      for (int rb = 0; rb < BK / 32; ++rb)
#pragma unroll
        for (int g = (rb == 0 ? 1 : 0); g < 4; g += 2)
          red = (g + 1 < 4) ? fmin3(red, mn[rb][g], mn[rb][g + 1]) : __builtin_fminf(red, mn[rb][g]);
      red = pair_min(red);
    }
    const float mt = red * cexp;
    const bool need = mt > m_run + ATTN_RESCALE_SLACK;
    if (wave_any(need)) {
      const float mnew = need ? mt : m_run;
      const float alpha = need ? fast_exp2(m_run - mnew) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
      m_run = mnew;
    }
  };
  // P = exp2(s*c - m_run) packed to bf16 into pb; returns this lane's sum
  // of the fp32 exponentials (the lse needs the unrounded normaliser)
  auto expsum = [&](const f32x16(&s)[BK / 32], auto masked) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
    const float nm = -m_run;
    float tsum = 0.f;
#pragma unroll
    for (int rb = 0; rb < BK / 32; ++rb) {
      float p[16];
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const float e = fast_exp2(__builtin_fmaf(s[rb][rr], cexp, nm));
        // a hidden score is +-inf; with c == 0 the product would be NaN, so select
        p[rr] = (MASKED && s[rb][rr] == maskval) ? 0.f : e;
      }
      pb[2 * rb] = pack8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
      pb[2 * rb + 1] = pack8(p[8], p[9], p[10], p[11], p[12], p[13], p[14], p[15]);
      float t8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) t8[i] = p[i] + p[i + 8];
      const float rs = ((t8[0] + t8[1]) + (t8[2] + t8[3])) + ((t8[4] + t8[5]) + (t8[6] + t8[7]));
      tsum = rb == 0 ? rs : tsum + rs;
    }
    return tsum;
  };
  auto softmax = [&](f32x16(&s)[BK / 32], auto masked) {
    if (ATTN_PF_LAZYMAX) {
      float tsum = expsum(s, masked);
      if (wave_any(!(tsum <= 4294967296.f))) {   // also true for inf and NaN
        raise_max(s);
        tsum = expsum(s, masked);
      }
      l_run += tsum;
    } else {
      raise_max(s);
      l_run += expsum(s, masked);
    }
  };

  // Two-group ping-pong.  Waves 0-3 (group A) and 4-7 (group B) share the
  // SIMDs pairwise (wave w and w + 4 run on the same SIMD).  Each tile takes
  // two phases separated by workgroup barriers; in every phase one group runs
  // its matrix work G(j) = [P.V of tile j-1, QK of tile j] while the other runs
  // its softmax of the tile it has just multiplied, so the exponentials of one
  // wave execute next to the MFMAs of its SIMD neighbour:
  //     phase 2j   : A G(j)      B softmax(j-1)
  //     phase 2j+1 : A softmax(j) B G(j)
  // K(j+1) and V(j) are fetched at the start of phase 2j and written to LDS at
  // the end of phase 2j+1 (double-buffered: K(j) and V(j-1) are read during
  // phases 2j and 2j+1).
  const bool grpA = w < C::NW / 2;
  auto active = [&](int jj) __attribute__((always_inline)) {
    return jj >= 0 && jj < nt && (j0 + jj) * BK < kend_w && (j0 + jj + 1) * BK > kbeg_w;
  };
  // hidden scores of tile jj set to maskval (tiles that cross the diagonal,
  // the end of the keys or a window's lower edge); true if it did
  auto mask_tile = [&](f32x16(&s)[BK / 32], int jj) __attribute__((always_inline)) {
    const int k0 = (j0 + jj) * BK;
    if (!(k0 + BK > kmask_from || k0 < klo_until)) return false;
    const int lim = a.causal ? min(a.Lk - 1, qrow + off) : a.Lk - 1;
#pragma unroll
    for (int rb = 0; rb < BK / 32; ++rb)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int key = k0 + 32 * rb + 8 * (rr >> 2) + 4 * hh + (rr & 3);
        s[rb][rr] = (key <= lim && key >= qlo) ? s[rb][rr] : maskval;
      }
    return true;
  };
  // S^T of tile jj: the QK MFMAs (their K operand reads ATTN_PF_QK_AHEAD
  // ahead), with the NLD direct loads of LOADS among them
  auto qk = [&](f32x16(&s)[BK / 32], const uint16_t *ks_, auto loads, auto nld) __attribute__((always_inline)) {
    constexpr int NLD = decltype(nld)::value;
    constexpr int N = (BK / 32) * (D / 16);
    constexpr int A = ATTN_PF_QK_AHEAD;
    constexpr int SP = NLD > 0 && N / (NLD > 0 ? NLD : 1) > 0 ? N / (NLD > 0 ? NLD : 1) : 1;
    auto kread = [&](int i) __attribute__((always_inline)) {
      const int rb = kPfAlt ? i % (BK / 32) : i / (D / 16), ks = kPfAlt ? i / (BK / 32) : i % (D / 16);
      return ld16(ks_ + 32 * rb * D + koff(ks));
    };
#pragma unroll
    for (int rb = 0; rb < BK / 32; ++rb) s[rb] = f32x16{};
    if (ATTN_PF_PIPE) {
      // as in pv: reads A MFMAs ahead in a ring, the order held by fences;
      // load i of LOADS follows MFMA i * SP
      u32x4 kr[A + 1];
#pragma unroll
      for (int i = 0; i < A && i < N; ++i) kr[i] = kread(i);
#pragma unroll
      for (int i = 0; i < N; ++i) {
        if (i + A < N) kr[(i + A) % (A + 1)] = kread(i + A);
        __builtin_amdgcn_sched_barrier(0);
        const int rb = kPfAlt ? i % (BK / 32) : i / (D / 16), ks = kPfAlt ? i / (BK / 32) : i % (D / 16);
        s[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kr[i % (A + 1)]), qf[ks], s[rb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (NLD > 0 && i % SP == 0 && i / SP < NLD) {
          loads(i / SP);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int rb = kPfAlt ? i % (BK / 32) : i / (D / 16), ks = kPfAlt ? i / (BK / 32) : i % (D / 16);
      s[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kread(i)), qf[ks], s[rb], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NLD; ++i) loads(i);
    __builtin_amdgcn_sched_group_barrier(0x100, A, 0);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (NLD > 0 && i % SP == 0 && i / SP < NLD) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
      if (i < N - A) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };

  f32x16 s[BK / 32];
  // LOADS (NLD direct loads, NLD > 0) go among the QK MFMAs, which then run
  // whether or not this wave sees tile jj (every wave must move its share of
  // the tiles; the scores of a tile it does not see are not used)
  auto gemm = [&](int jj, const uint16_t *ks_, const uint16_t *vs_, auto loads, auto nld)
      __attribute__((always_inline)) {
    constexpr int NLD = decltype(nld)::value;
    if (active(jj - 1)) pv(vs_);
    if (NLD > 0 || active(jj))
      qk(s, ks_, loads, nld);
  };
  auto soft = [&](int jj) __attribute__((always_inline)) {
    if (!active(jj)) return;
    if (mask_tile(s, jj)) softmax(s, std::true_type{});
    else softmax(s, std::false_type{});
  };

  // One tile step j (P = j % 2): K(j) is in kb[P], V(j-1) in vb[1-P].
  // Group A runs its matrix work G(j) = [P.V of tile j-1, QK of tile j], with
  // the direct loads of K(j+1) into kb[1-P] and V(j) into vb[P] spread over
  // its QK MFMAs, then the softmax of tile j.  Group B runs the softmax of
  // tile j-1, then G(j).  So the exponentials of one wave execute next to the
  // MFMAs of its SIMD neighbour, and no wave stalls on a burst of loads (a
  // direct load holds its wave until the CU's address unit takes it).  Both
  // target buffers were last read in step j-1.  The step ends with every
  // wave's loads complete and a workgroup barrier, which publishes them.
  auto step = [&](int j, auto parity) __attribute__((always_inline)) {
    constexpr int P = decltype(parity)::value;
    uint16_t *kcur = P ? kb1 : kb0;
    uint16_t *knext = P ? kb0 : kb1;
    uint16_t *vprev = P ? vb0 : vb1;
    uint16_t *vcur = P ? vb1 : vb0;
    auto none = [](int) __attribute__((always_inline)) {};
    constexpr auto n0 = std::integral_constant<int, 0>{};
    if (grpA) {
      __builtin_amdgcn_s_setprio(kPrioGemm);
      // K(j+1) and V(j) among the QK MFMAs (past the last tile: a repeat of
      // it, never read)
#if ATTN_DEVICE_PASS
      const auto rk = tile_rs(kg, j0 + max(0, min(j + 1, nt - 1)));
      const auto rv = tile_rs(vg, j0 + max(0, min(j, nt - 1)));
      gemm(j, kcur, vprev, [&](int i) __attribute__((always_inline)) {
        if (i < 2 * C::DPW) dma_one(rk, knext, i, std::false_type{});
        else dma_one(rv, vcur, i - 2 * C::DPW, std::true_type{});
      }, std::integral_constant<int, 4 * C::DPW>{});
#else
      gemm(j, kcur, vprev, none, std::integral_constant<int, 4 * C::DPW>{});
#endif
      __builtin_amdgcn_s_setprio(kPrioSoft);
      soft(j);
    } else {
      __builtin_amdgcn_s_setprio(kPrioSoft);
      soft(j - 1);
      __builtin_amdgcn_s_setprio(kPrioGemm);
      gemm(j, kcur, vprev, none, n0);
    }
    __builtin_amdgcn_s_setprio(0);
    ATTN_WAIT_VMEM();
    __syncthreads();
  };

  if (nt > 0 && grpA) dma(kg, kb0, j0, std::false_type{});
  ATTN_WAIT_VMEM();
  __syncthreads();
  for (int j = 0; j <= nt; j += 2) {
    step(j, std::integral_constant<int, 0>{});
    if (j + 1 > nt) break;
    step(j + 1, std::integral_constant<int, 1>{});
  }

  // ---- epilogue: out = O / l, lse = m ln2 + ln l -------------------------
  const float lt = pair_sum(l_run);
  if (qrow < a.Lq && a.nsplit == 1) {
    const float inv = 1.f / lt;
    uint16_t *op = a.out + (((size_t)b * a.Hq + head) * a.Lq + qrow) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 v4;
        v4[0] = (__bf16)(o[db][4 * g4 + 0] * inv);
        v4[1] = (__bf16)(o[db][4 * g4 + 1] * inv);
        v4[2] = (__bf16)(o[db][4 * g4 + 2] * inv);
        v4[3] = (__bf16)(o[db][4 * g4 + 3] * inv);
        *reinterpret_cast<bf16x4 *>(op + 32 * db + 8 * g4 + 4 * hh) = v4;
      }
    }
    if (a.lse != nullptr && hh == 0)
      a.lse[((size_t)b * a.Hq + head) * a.Lq + qrow] = m_run * ATTN_LN2 + __logf(lt);
  } else if (qrow < a.Lq) {
    // one key range of several: its normalised output and log-sum-exp (a row
    // that sees no key of this range has l = 0: output 0, lse -inf)
    const size_t row = ((size_t)b * a.Hq + head) * a.Lq + qrow;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    float *po = a.part_o + (row * a.nsplit + sp) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 v4 = {o[db][4 * g4] * inv, o[db][4 * g4 + 1] * inv, o[db][4 * g4 + 2] * inv,
                          o[db][4 * g4 + 3] * inv};
        *reinterpret_cast<f32x4 *>(po + 32 * db + 8 * g4 + 4 * hh) = v4;
      }
    }
    if (hh == 0) a.part_lse[row * a.nsplit + sp] = lt > 0.f ? m_run * ATTN_LN2 + __logf(lt) : -__builtin_inff();
  }
  }  // work items
}

// In-wave pipelined variant.  Every wave runs the same schedule; per tile j
// (keys of tile j in S^T registers `cur`):
//   barrier; direct loads of K(j+2) and V(j+1) into the buffers freed by the
//   barrier; mask and tile maximum of tile j, running-max raise;
//   bracket 1: MFMA  S^T(j+1) = K(j+1) Q^T             VALU  P(j) = exp2(S c - m)
//   bracket 2: MFMA  O^T += V(j)^T P(j)^T               VALU  row sum of P(j)
// Within a bracket the matrix and vector work are independent, and
// sched_group_barrier interleaves them, so the exponentials run while the
// matrix core works on the same wave's products; the second wave of the SIMD
// fills what is left.  K(t) sits in kb[t % 2], V(t) in vb[t % 2].
template <int D, int BK>
__global__ __launch_bounds__(kPfThreads<D>) void prefill_iw_kernel(PrefillArgs a) {
  using C = PrefillCfg<D, BK>;
  __shared__ __attribute__((aligned(1024))) uint16_t kb0[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t kb1[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t vb0[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t vb1[C::TILE];

  // ---- which tile: XCD-grouped, heaviest q-block first; one work item per
  // workgroup or, for head dims built with resident workgroups and
  // a.persist > 0, several per workgroup (as in prefill_kernel) ------------
  const int tf = a.total & ~7;
  auto item = [&](int t) __attribute__((always_inline)) {
  const int sp = t % a.nsplit;
  t /= a.nsplit;
  int unit = t / a.n_qblk;
  const int r = t - unit * a.n_qblk;
  const int qblk = a.causal ? (a.n_qblk - 1 - r) : r;
  const int hg = unit % a.n_hg;
  unit /= a.n_hg;
  const int hkv = unit % a.Hkv;
  const int b = unit / a.Hkv;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int ql = lane & 31, hh = lane >> 5;
  const int head = hkv * a.G + hg * a.hpw + w / a.wph;
  const int q0w = qblk * a.Bq + (w % a.wph) * 32;
  const int qrow = q0w + ql;
  const int off = a.Lk - a.Lq;

  const int qlast_wg = min(qblk * a.Bq + a.Bq, a.Lq) - 1;
  const int kend_wg = a.causal ? min(a.Lk, qlast_wg + off + 1) : a.Lk;
  const int kmask_from = a.causal ? min(a.Lk, q0w + off + 1) : a.Lk;
  const int win = a.window;
  const int kbeg_wg = win ? max(0, qblk * a.Bq + off - win + 1) : 0;
  const int klo_until = win ? q0w + 31 + off - win + 1 : 0;
  const int qlo = win ? qrow + off - win + 1 : -0x7fffffff;
  const int jbeg = kbeg_wg / BK;
  const int nt_all = (kend_wg + BK - 1) / BK - jbeg;
  const int j0 = jbeg + (int)((long long)nt_all * sp / a.nsplit);
  const int nt = jbeg + (int)((long long)nt_all * (sp + 1) / a.nsplit) - j0;

  const int qr = min(qrow, a.Lq - 1);
  const uint16_t *qp = a.q + (((size_t)b * a.Hq + head) * a.Lq + qr) * D;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) qf[ks] = as_bf16x8(ld16(qp + 16 * ks + 8 * hh));

  const size_t kvoff = ((size_t)b * a.Hkv + hkv) * (size_t)a.Lk * D;
  const uint16_t *kg = a.k + kvoff;
  const uint16_t *vg = a.v + kvoff;

  // tile j of K or V into LDS: every wave moves DPW blocks of 1 KiB
  auto dma = [&](const uint16_t *g, uint16_t *dst, int j, auto is_v) __attribute__((always_inline)) {
    constexpr bool V = decltype(is_v)::value;
#if ATTN_DEVICE_PASS
    const auto rs = buf_rsrc_uniform(g + (size_t)j * BK * D, (uint32_t)min(BK, a.Lk - j * BK) * (D * 2));
#pragma unroll
    for (int i = 0; i < C::DPW; ++i) {
      const int blk = wu * C::DPW + i;
      const int row = blk * C::RPD + lane / C::CPR;
      const int c = (lane % C::CPR) ^ (V ? vswz<D>(row) : kswz<D>(row));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t *)(dst + blk * 512), 16,
                                               (lane / C::CPR) * (D * 2) + 16 * c, blk * 1024, 0, 0);
    }
#endif
  };

  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = f32x16{};
  // The running maximum starts at the lowest finite float, not -inf, so that
  // a tile whose scores are all hidden gives exp2(-inf - m) = 0 rather than
  // NaN: every tile of the workgroup's range goes through the same steps,
  // and one a row does not see contributes exactly zero.  The first visible
  // score raises it (any finite value exceeds it).
  float m_run = -3.40282347e38f;
  float l_run = 0.f;
  // A hidden score is -inf (c > 0) or +inf (c < 0), so exp2(s c - m) is
  // exactly 0 for it with no select.  c = 0 would give 0 * inf = NaN; the
  // smallest normal float stands in for it: every visible weight
  // exp2(s c - m) still rounds to exactly 1.
  const float cexp = a.c == 0.f ? 1.17549435e-38f : a.c;
  const bool cpos = cexp >= 0.f;
  const float maskval = cpos ? -__builtin_inff() : __builtin_inff();

  const int g16 = lane >> 4, j16 = lane & 15;
  constexpr int NKO = D / 16 < 8 ? D / 16 : 8;
  constexpr int NVO = D / 32 < 4 ? D / 32 : 4;
  int koffs[NKO];
#pragma unroll
  for (int ks = 0; ks < NKO; ++ks) koffs[ks] = ql * D + 8 * ((2 * ks + hh) ^ kswz<D>(ql));
  int voffs[NVO];
  {
    const int vr = 4 * hh + (j16 >> 2);
    const int tv = vswz<D>(vr) >> 2;
    const int cin = 2 * (g16 & 1) + ((j16 & 3) >> 1);
#pragma unroll
    for (int db = 0; db < NVO; ++db) voffs[db] = vr * D + 8 * (4 * (db ^ tv) + cin) + 4 * (j16 & 1);
  }
  auto koff = [&](int ks) __attribute__((always_inline)) { return koffs[ks % NKO] + (ks / NKO) * 128; };
  auto voff = [&](int db) __attribute__((always_inline)) { return voffs[db % NVO] + (db / NVO) * 128; };

  bf16x8 pb[BK / 16];
  constexpr int NQK = (BK / 32) * (D / 16);  // MFMAs of S^T per tile
  constexpr int NPV = (D / 32) * (BK / 16);  // MFMAs of O^T per tile

  auto qk_ops = [&](f32x16(&s)[BK / 32], const uint16_t *ks_) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < BK / 32; ++rb) s[rb] = f32x16{};
#pragma unroll
    for (int i = 0; i < (BK / 32) * (D / 16); ++i) {
      const int rb = kIwAlt ? i % (BK / 32) : i / (D / 16), ks = kIwAlt ? i / (BK / 32) : i % (D / 16);
      s[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ld16(ks_ + 32 * rb * D + koff(ks))), qf[ks], s[rb],
                                                      0, 0, 0);
    }
  };
  auto pv_ops = [&](const uint16_t *vs_) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < (D / 32) * (BK / 16); ++i) {
      const int db = kIwAlt ? i % (D / 32) : i / (BK / 16), kb = kIwAlt ? i / (D / 32) : i % (BK / 16);
      const uint16_t *vp = vs_ + 16 * kb * D + voff(db);
      const bf16x4 lo = lds_tr16(vp);
      const bf16x4 hi = lds_tr16(vp + 8 * D);
      const bf16x8 vop = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb[kb], o[db], 0, 0, 0);
    }
  };
  // P = exp2(s c - m) in place (s keeps the fp32 values for the row sum), packed to bf16 in pb
  auto expo = [&](f32x16(&s)[BK / 32]) __attribute__((always_inline)) {
    const float nm = -m_run;
#pragma unroll
    for (int rb = 0; rb < BK / 32; ++rb) {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) s[rb][rr] = fast_exp2(__builtin_fmaf(s[rb][rr], cexp, nm));
      pb[2 * rb] = pack8(s[rb][0], s[rb][1], s[rb][2], s[rb][3], s[rb][4], s[rb][5], s[rb][6], s[rb][7]);
      pb[2 * rb + 1] = pack8(s[rb][8], s[rb][9], s[rb][10], s[rb][11], s[rb][12], s[rb][13], s[rb][14], s[rb][15]);
    }
  };
  // P = exp2(s c - m) packed to bf16 in pb, the scores kept; returns this
  // lane's sum of the fp32 exponentials
  auto expo_sum = [&](const f32x16(&s)[BK / 32]) __attribute__((always_inline)) {
    const float nm = -m_run;
    float tsum = 0.f;
#pragma unroll
    for (int rb = 0; rb < BK / 32; ++rb) {
      float p[16];
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) p[rr] = fast_exp2(__builtin_fmaf(s[rb][rr], cexp, nm));
      pb[2 * rb] = pack8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
      pb[2 * rb + 1] = pack8(p[8], p[9], p[10], p[11], p[12], p[13], p[14], p[15]);
      float t8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) t8[i] = p[i] + p[i + 8];
      const float rs = ((t8[0] + t8[1]) + (t8[2] + t8[3])) + ((t8[4] + t8[5]) + (t8[6] + t8[7]));
      tsum = rb == 0 ? rs : tsum + rs;
    }
    return tsum;
  };
  auto rsum = [&](const f32x16(&s)[BK / 32]) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < BK / 32; ++rb) {
      float t8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) t8[i] = s[rb][i] + s[rb][i + 8];
      l_run += ((t8[0] + t8[1]) + (t8[2] + t8[3])) + ((t8[4] + t8[5]) + (t8[6] + t8[7]));
    }
  };
  // hidden scores of tile j set to maskval (tiles that cross the diagonal, the
  // end of the keys or the window's lower edge)
  auto mask_tile = [&](f32x16(&s)[BK / 32], int jj) __attribute__((always_inline)) {
    const int k0 = (j0 + jj) * BK;
    if (!uniform(k0 + BK > kmask_from || k0 < klo_until)) return;
    const int lim = a.causal ? min(a.Lk - 1, qrow + off) : a.Lk - 1;
#pragma unroll
    for (int rb = 0; rb < BK / 32; ++rb)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int key = k0 + 32 * rb + 8 * (rr >> 2) + 4 * hh + (rr & 3);
        s[rb][rr] = (key <= lim && key >= qlo) ? s[rb][rr] : maskval;
      }
  };
  // raise the running maximum to the tile's if it exceeds it by more than the slack
  auto raise = [&](const f32x16(&s)[BK / 32]) __attribute__((always_inline)) {
    float red;
    if (cpos) {
      red = s[0][0];
#pragma unroll
      for (int rb = 0; rb < BK / 32; ++rb)
#pragma unroll
        for (int g = 0; g < 16; g += 2) {
          if (rb == 0 && g == 0) red = __builtin_fmaxf(s[0][0], s[0][1]);
          else red = fmax3(red, s[rb][g], s[rb][g + 1]);
        }
      red = pair_max(red);
    } else {
      red = s[0][0];
#pragma unroll
      for (int rb = 0; rb < BK / 32; ++rb)
#pragma unroll
        for (int g = 0; g < 16; g += 2) {
          if (rb == 0 && g == 0) red = __builtin_fminf(s[0][0], s[0][1]);
          else red = fmin3(red, s[rb][g], s[rb][g + 1]);
        }
      red = pair_min(red);
    }
    const float mt = red * cexp;
    const bool need = mt > m_run + ATTN_RESCALE_SLACK;
    if (wave_any(need)) {
      const float mnew = need ? mt : m_run;
      const float alpha = need ? fast_exp2(m_run - mnew) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        // D = 256: O lives in AGPRs (accumulation registers), which vector
        // arithmetic cannot address; the empty asm statements, which take O
        // in AGPRs, keep its copies to and from vector registers inside this
        // rarely taken branch (without them the compiler placed 128 such
        // copies per tile on the common path)
        if constexpr (D == 256) asm volatile("" : "+a"(o[db]));
        o[db] *= alpha;
        if constexpr (D == 256) asm volatile("" : "+a"(o[db]));
      }
      m_run = mnew;
    }
  };

  // interleave orders: K reads ATTN_PF_QK_AHEAD ahead, V^T reads ATTN_PF_PV_AHEAD ahead;
  // bracket 1 also carries the direct loads of the next tiles, one every SP
  // MFMAs (a direct load holds its wave until the CU's address unit takes it,
  // about 1 KiB per 16 cycles per CU, so loads issued together stall every wave)
  constexpr bool SPREAD = (ATTN_PF_IW_SPREAD & (D == 64 ? 1 : D == 128 ? 2 : 4)) != 0;
  constexpr int NLD = SPREAD ? 2 * C::DPW : 0;
  constexpr int SP = NLD ? (NQK / NLD > 0 ? NQK / NLD : 1) : 1;
  auto sched_b1 = [&]() __attribute__((always_inline)) {
    constexpr int A = D == 256 ? ATTN_PF_IW_QKA256 : ATTN_PF_QK_AHEAD;
    constexpr int V1 = D == 256 ? ATTN_PF_IW_V1_256 : ATTN_PF_IW_V1;
    __builtin_amdgcn_sched_group_barrier(0x100, A, 0);
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, V1, 0);
      if (NLD && i % SP == 0 && i / SP < NLD) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
      if (i < NQK - A) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };
  auto sched_b2 = [&]() __attribute__((always_inline)) {
    constexpr int A = D == 256 ? ATTN_PF_IW_PVA256 : ATTN_PF_PV_AHEAD;
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * A, 0);
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, ATTN_PF_IW_V2, 0);
      if (i < NPV - A) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  };

  // one tile: see the comment above the kernel
  auto iter = [&](int j, auto parity, f32x16(&cur)[BK / 32], f32x16(&nxt)[BK / 32]) __attribute__((always_inline)) {
    constexpr int P = decltype(parity)::value;
    uint16_t *kread = P ? kb0 : kb1;  // K(j+1)
    uint16_t *kfill = P ? kb1 : kb0;  // K(j+2)
    uint16_t *vread = P ? vb1 : vb0;  // V(j)
    uint16_t *vfill = P ? vb0 : vb1;  // V(j+1)
    ATTN_WAIT_VMEM();
    __syncthreads();
    if (!SPREAD) {
      if (j + 2 < nt) dma(kg, kfill, j0 + j + 2, std::false_type{});
      if (j + 1 < nt) dma(vg, vfill, j0 + j + 1, std::true_type{});
    }
    mask_tile(cur, j);
    if (ATTN_PF_IW_LAZY && D < 256) {   // (D = 256: the 32 exponential registers would spill)
      // bracket 1: exponentials of tile j against the running max, and their
      // row sums, beside the products of tile j+1 and the direct loads; the
      // tile maximum is taken (and the tile exponentiated again) only when
      // some sum exceeds 2^32 or is not finite, as in prefill_kernel
      float tsum = expo_sum(cur);
      qk_ops(nxt, kread);
      if (SPREAD) {
        dma(kg, kfill, j0 + min(j + 2, nt - 1), std::false_type{});
        dma(vg, vfill, j0 + min(j + 1, nt - 1), std::true_type{});
      }
      sched_b1();
      __builtin_amdgcn_sched_barrier(0);
      if (wave_any(!(tsum <= 4294967296.f))) {
        raise(cur);
        tsum = expo_sum(cur);
      }
      l_run += tsum;
      // bracket 2: P.V of tile j
      pv_ops(vread);
      sched_b2();
      return;
    }
    raise(cur);
    // bracket 1: exponentials of tile j beside the products of tile j+1 (past
    // the last tile those products are not used) and the direct loads of
    // K(j+2) and V(j+1) (past the last tile they repeat it: never read)
    expo(cur);
    qk_ops(nxt, kread);
    if (SPREAD) {
      dma(kg, kfill, j0 + min(j + 2, nt - 1), std::false_type{});
      dma(vg, vfill, j0 + min(j + 1, nt - 1), std::true_type{});
    }
    sched_b1();
    __builtin_amdgcn_sched_barrier(0);
    // bracket 2: P.V of tile j beside its row sums
    pv_ops(vread);
    rsum(cur);
    sched_b2();
  };

  f32x16 sa[BK / 32], sb[BK / 32];
  if (nt > 0) {
    dma(kg, kb0, j0, std::false_type{});
    dma(vg, vb0, j0, std::true_type{});
    if (nt > 1) dma(kg, kb1, j0 + 1, std::false_type{});
  }
  ATTN_WAIT_VMEM();
  __syncthreads();
  qk_ops(sa, kb0);
  for (int j = 0; j < nt; j += 2) {
    iter(j, std::integral_constant<int, 0>{}, sa, sb);
    if (j + 1 >= nt) break;
    iter(j + 1, std::integral_constant<int, 1>{}, sb, sa);
  }

  // ---- epilogue: out = O / l, lse = m ln2 + ln l -------------------------
  const float lt = pair_sum(l_run);
  if (qrow < a.Lq && a.nsplit == 1) {
    const float inv = 1.f / lt;
    uint16_t *op = a.out + (((size_t)b * a.Hq + head) * a.Lq + qrow) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 v4;
        v4[0] = (__bf16)(o[db][4 * g4 + 0] * inv);
        v4[1] = (__bf16)(o[db][4 * g4 + 1] * inv);
        v4[2] = (__bf16)(o[db][4 * g4 + 2] * inv);
        v4[3] = (__bf16)(o[db][4 * g4 + 3] * inv);
        *reinterpret_cast<bf16x4 *>(op + 32 * db + 8 * g4 + 4 * hh) = v4;
      }
    }
    if (a.lse != nullptr && hh == 0)
      a.lse[((size_t)b * a.Hq + head) * a.Lq + qrow] = m_run * ATTN_LN2 + __logf(lt);
  } else if (qrow < a.Lq) {
    const size_t row = ((size_t)b * a.Hq + head) * a.Lq + qrow;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    float *po = a.part_o + (row * a.nsplit + sp) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 v4 = {o[db][4 * g4] * inv, o[db][4 * g4 + 1] * inv, o[db][4 * g4 + 2] * inv,
                          o[db][4 * g4 + 3] * inv};
        *reinterpret_cast<f32x4 *>(po + 32 * db + 8 * g4 + 4 * hh) = v4;
      }
    }
    if (hh == 0) a.part_lse[row * a.nsplit + sp] = lt > 0.f ? m_run * ATTN_LN2 + __logf(lt) : -__builtin_inff();
  }
  };
  if constexpr (kPersist<D>) {
    const int per_x = tf >> 3, q8 = a.persist >> 3;
    const int px = blockIdx.x & 7, pi = blockIdx.x >> 3;
    bool tail_done = false;
    for (int it = 0;; ++it) {
      int t;
      if (a.persist == 0) {
        if (it > 0) break;
        t = blockIdx.x;
        if (t < tf) t = (t & 7) * per_x + (t >> 3);
      } else {
        const int kx = it * q8 + ((it & 1) ? q8 - 1 - pi : pi);
        if (kx < per_x) {
          t = px * per_x + kx;
        } else if (!tail_done && (int)blockIdx.x < a.total - tf) {
          t = tf + blockIdx.x;
          tail_done = true;
        } else {
          break;
        }
      }
      item(t);
    }
  } else {
    int t = blockIdx.x;
    if (t < tf) t = (t & 7) * (tf >> 3) + (t >> 3);
    item(t);
  }
}

// Merge of the key ranges of one query row (one wave per row, nsplit <= 64):
// lse = log sum_s exp(lse_s), out = sum_s exp(lse_s - lse) out_s.  This is the
// softmax sum split over disjoint key sets.
template <int D>
__global__ __launch_bounds__(256) void prefill_combine_kernel(PrefillArgs a, long long rows) {
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const int S = a.nsplit;
  const float lv = lane < S ? a.part_lse[row * S + lane] : -__builtin_inff();
  float mx = lv;
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, sh));
  const float wgt = (lane < S && lv > -__builtin_inff()) ? fast_exp2((lv - mx) * ATTN_LOG2E) : 0.f;
  float den = wgt;
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) den += __shfl_xor(den, sh);
  constexpr int PER = D / 64;
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  const float *po = a.part_o + (size_t)row * S * D + lane * PER;
  int s = 0;
  // four ranges' loads issued together (every range wrote its partial),
  // then added in range order
  for (; s + 4 <= S; s += 4) {
    float x[4][PER];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < PER; ++i) x[u][i] = po[(size_t)(s + u) * D + i];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float ws = __shfl(wgt, s + u);
      if (ws != 0.f) {
#pragma unroll
        for (int i = 0; i < PER; ++i) acc[i] += ws * x[u][i];
      }
    }
  }
  for (; s < S; ++s) {
    const float ws = __shfl(wgt, s);
    if (ws != 0.f) {
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[i] += ws * po[(size_t)s * D + i];
    }
  }
  const float inv = 1.f / den;
  uint16_t *op = a.out + (size_t)row * D + lane * PER;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const __bf16 h = (__bf16)(acc[i] * inv);
    op[i] = __builtin_bit_cast(uint16_t, h);
  }
  if (a.lse != nullptr && lane == 0) a.lse[row] = mx + __logf(den);
}

// whether head dim D runs on prefill_iw_kernel (else prefill_kernel); only
// the kernel a head dim uses is instantiated
template <int D>
constexpr bool kUseIw = (ATTN_PF_IW & (D == 64 ? 1 : D == 128 ? 2 : 4)) != 0;

template <int D, int BK>
static hipError_t launch_t(const PrefillArgs &a, hipStream_t s) {
  if constexpr (kUseIw<D>)
    hipLaunchKernelGGL((prefill_iw_kernel<D, BK>), dim3(a.persist > 0 ? a.persist : a.total),
                       dim3(PrefillCfg<D, BK>::NT), 0, s, a);
  else
    hipLaunchKernelGGL((prefill_kernel<D, BK>), dim3(a.persist > 0 ? a.persist : a.total),
                       dim3(PrefillCfg<D, BK>::NT), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  const long long rows = (long long)a.B * a.Hq * a.Lq;
  hipLaunchKernelGGL((prefill_combine_kernel<D>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a, rows);
  return hipGetLastError();
}

bool prefill_can_persist(int D) {
  switch (D) {
    case 64: return kPersist<64>;
    case 128: return kPersist<128>;
    case 256: return kPersist<256>;
    default: return false;
  }
}

int prefill_tile_keys(int D) { return D == 256 ? ATTN_PF_BK256 : (D == 128 ? ATTN_PF_BK128 : 64); }

// Query-row packing of the kernel above: 8 waves x 32 rows per workgroup.
bool prefill_plan(PrefillArgs &a, int D) {
  const int nw = D == 256 ? PrefillCfg<256, ATTN_PF_BK256>::NW : 8;
  const int rows = 32;
  int g = a.G, x = nw;
  while (x) {
    const int t = g % x;
    g = x;
    x = t;
  }
  a.hpw = g;                       // query heads per workgroup: gcd(G, waves)
  a.wph = nw / a.hpw;              // waves per head
  a.Bq = rows * a.wph;             // query rows per head per workgroup
  a.n_qblk = (a.Lq + a.Bq - 1) / a.Bq;
  a.n_hg = a.G / a.hpw;
  const long long total = (long long)a.n_qblk * a.Hkv * a.n_hg * a.B * a.nsplit;
  if (total > 0x7fffffffLL) return false;
  a.total = (int)total;
  return true;
}

template <int D, int BK>
static hipError_t wgs_per_cu_t(int *out) {
  const void *f;
  if constexpr (kUseIw<D>) f = (const void *)&prefill_iw_kernel<D, BK>;
  else f = (const void *)&prefill_kernel<D, BK>;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(out, f, PrefillCfg<D, BK>::NT, 0);
}

hipError_t prefill_wgs_per_cu(int D, int *out) {
  switch (D) {
    case 64: return wgs_per_cu_t<64, 64>(out);
    case 128: return wgs_per_cu_t<128, ATTN_PF_BK128>(out);
    case 256: return wgs_per_cu_t<256, ATTN_PF_BK256>(out);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prefill(const PrefillArgs &a, int D, hipStream_t s) {
  switch (D) {
    case 64: return launch_t<64, 64>(a, s);
    case 128: return launch_t<128, ATTN_PF_BK128>(a, s);
    case 256: return launch_t<256, ATTN_PF_BK256>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
