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
//  * One workgroup = 4 wave64s = 128 query rows of up to 4 query heads that
//    share one KV head; every K/V tile it stages in LDS serves all of them.
//  * Each wave owns 32 query rows and computes the transposed score block
//    S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (keys on the M side, queries on
//    the N side).  In the accumulator layout a lane holds one query column and
//    16 keys per 32-key block, so row max / row sum are lane-local plus one
//    exchange between the two wave halves.
//  * P^T (bf16) is fed to O^T += V^T P^T straight from those registers: the
//    16 keys a lane holds for one P.V step are the same keys its V^T operand
//    reads, because V^T is written to LDS with the matching key order.
//  * V is transposed once per tile on its way into LDS (4 keys x 8 dims per
//    thread, byte permutes), K is copied as is; both double-buffered.
//  * Softmax in the log2 domain: p = exp2(s*c - m) with c = scale*log2(e);
//    the running maximum is raised lazily (ATTN_RESCALE_SLACK), so the O
//    rescale is skipped on almost every tile.
//  * Causal: tiles past a wave's last visible key are skipped, the mask is
//    evaluated only on tiles that cross the diagonal or the end of the keys.
//    Workgroups are issued heaviest first, and consecutive workgroup ids are
//    spread over the 8 XCDs so that each XCD works on one KV head at a time
//    (its K/V stay in that XCD's L2).
#include "common.h"
#include "kernels.h"

namespace attn {

template <int D, int BK>
struct PrefillCfg {
  static constexpr int NW = 4;
  static constexpr int NT = NW * 64;
  static constexpr int KS = D + 8;       // K row stride in LDS (bf16 elements)
  static constexpr int VS = BK + 8;      // V^T row stride in LDS
  static constexpr int K_ELEMS = BK * KS;
  static constexpr int V_ELEMS = D * VS;
  static constexpr int BUF = K_ELEMS + V_ELEMS;
  static constexpr int K_CHUNKS = BK * D / 8;          // 16-byte pieces of a K tile
  static constexpr int K_PER_T = (K_CHUNKS + NT - 1) / NT;
  static constexpr int V_UNITS = (BK / 4) * (D / 8);    // 4 keys x 8 dims each
  static constexpr int V_PER_T = (V_UNITS + NT - 1) / NT;
  static_assert(BK % 32 == 0 && D % 32 == 0, "tile shape");
};

// Position of key k (0..15 inside a 16-key group) in the V^T row: the lane
// half hh reads positions 8*hh..8*hh+7, which must be keys
// {4hh..4hh+3, 8+4hh..8+4hh+3}, the keys the S^T accumulator gives that half.
ATTN_DEV int vt_pos16(int k16) { return 8 * ((k16 >> 2) & 1) + 4 * (k16 >> 3) + (k16 & 3); }

template <int D, int BK>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillArgs a) {
  using C = PrefillCfg<D, BK>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * C::BUF];

  // ---- which tile: XCD-grouped, heaviest q-block first -------------------
  const int bid = blockIdx.x;
  int t = bid;
  const int tf = a.total & ~7;
  if (bid < tf) t = (bid & 7) * (tf >> 3) + (bid >> 3);
  int unit = t / a.n_qblk;
  const int r = t - unit * a.n_qblk;
  const int qblk = a.causal ? (a.n_qblk - 1 - r) : r;
  const int hg = unit % a.n_hg;
  unit /= a.n_hg;
  const int hkv = unit % a.Hkv;
  const int b = unit / a.Hkv;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
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
  const int nt = (kend_wg + BK - 1) / BK;

  // ---- Q (B operand of S^T), kept in registers ----------------------------
  const int qr = min(qrow, a.Lq - 1);
  const uint16_t *qp = a.q + (((size_t)b * a.Hq + head) * a.Lq + qr) * D;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) qf[ks] = as_bf16x8(ld16(qp + 16 * ks + 8 * hh));

  const size_t kvoff = ((size_t)b * a.Hkv + hkv) * (size_t)a.Lk * D;
  const uint16_t *kg = a.k + kvoff;
  const uint16_t *vg = a.v + kvoff;

  u32x4 kreg[C::K_PER_T];
  u32x4 vreg[C::V_PER_T][4];
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  auto load_tile = [&](int j) {
    const int k0 = j * BK;
#pragma unroll
    for (int i = 0; i < C::K_PER_T; ++i) {
      const int c = tid + i * C::NT;
      if (C::K_CHUNKS % C::NT == 0 || c < C::K_CHUNKS) {
        const int key = c / (D / 8), dc = c % (D / 8);
        const int gk = k0 + key;
        kreg[i] = gk < a.Lk ? ld16(kg + (size_t)gk * D + dc * 8) : zero4;
      }
    }
#pragma unroll
    for (int i = 0; i < C::V_PER_T; ++i) {
      const int u = tid + i * C::NT;
      if (C::V_UNITS % C::NT == 0 || u < C::V_UNITS) {
        const int quad = u / (D / 8), dc = u % (D / 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int gk = k0 + 4 * quad + e;
          vreg[i][e] = gk < a.Lk ? ld16(vg + (size_t)gk * D + dc * 8) : zero4;
        }
      }
    }
  };

  auto store_tile = [&](int buf) {
    uint16_t *ks_ = smem + buf * C::BUF;
    uint16_t *vt = ks_ + C::K_ELEMS;
#pragma unroll
    for (int i = 0; i < C::K_PER_T; ++i) {
      const int c = tid + i * C::NT;
      if (C::K_CHUNKS % C::NT == 0 || c < C::K_CHUNKS) {
        const int key = c / (D / 8), dc = c % (D / 8);
        st16(ks_ + key * C::KS + dc * 8, kreg[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < C::V_PER_T; ++i) {
      const int u = tid + i * C::NT;
      if (C::V_UNITS % C::NT == 0 || u < C::V_UNITS) {
        const int quad = u / (D / 8), dc = u % (D / 8);
        const int k = 4 * quad;
        const int pos = (k & ~15) + vt_pos16(k & 15);
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) {
          const uint32_t a0 = vreg[i][0][w4], a1 = vreg[i][1][w4], a2 = vreg[i][2][w4], a3 = vreg[i][3][w4];
          u32x2 lo, hi;
          lo[0] = pack_lo16(a0, a1); lo[1] = pack_lo16(a2, a3);
          hi[0] = pack_hi16(a0, a1); hi[1] = pack_hi16(a2, a3);
          *reinterpret_cast<u32x2 *>(vt + (dc * 8 + 2 * w4) * C::VS + pos) = lo;
          *reinterpret_cast<u32x2 *>(vt + (dc * 8 + 2 * w4 + 1) * C::VS + pos) = hi;
        }
      }
    }
  };

  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = f32x16{};
  float m_run = -__builtin_inff();
  float l_run = 0.f;
  const float cexp = a.c;
  const bool cpos = cexp >= 0.f;
  const float maskval = cpos ? -__builtin_inff() : __builtin_inff();

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < nt; ++j) {
    if (j + 1 < nt) load_tile(j + 1);
    const uint16_t *ks_ = smem + (j & 1) * C::BUF;
    const uint16_t *vt = ks_ + C::K_ELEMS;
    const int k0 = j * BK;
    if (k0 < kend_w) {
      // S^T = K Q^T for BK keys x 32 queries
      f32x16 s[BK / 32];
#pragma unroll
      for (int rb = 0; rb < BK / 32; ++rb) {
        s[rb] = f32x16{};
        const uint16_t *kr = ks_ + (32 * rb + ql) * C::KS + 8 * hh;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
          s[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ld16(kr + 16 * ks)), qf[ks], s[rb], 0, 0, 0);
      }
      const bool need_mask = (k0 + BK > kmask_from);
      uint32_t vis[BK / 32];
      if (need_mask) {
        const int lim = a.causal ? min(a.Lk - 1, qrow + off) : a.Lk - 1;
#pragma unroll
        for (int rb = 0; rb < BK / 32; ++rb) {
          uint32_t bits = 0;
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            const int key = k0 + 32 * rb + 8 * (rr >> 2) + 4 * hh + (rr & 3);
            const bool vv = key <= lim;
            bits |= (vv ? 1u : 0u) << rr;
            s[rb][rr] = vv ? s[rb][rr] : maskval;
          }
          vis[rb] = bits;
        }
      }
      // tile maximum of s*c for this lane's query
      float red = s[0][0];
      if (cpos) {
#pragma unroll
        for (int rb = 0; rb < BK / 32; ++rb)
#pragma unroll
          for (int rr = (rb == 0 ? 1 : 0); rr < 16; rr += 2)
            red = (rr + 1 < 16) ? fmax3(red, s[rb][rr], s[rb][rr + 1]) : __builtin_fmaxf(red, s[rb][rr]);
        red = __builtin_fmaxf(red, xor32(red));
      } else {
#pragma unroll
        for (int rb = 0; rb < BK / 32; ++rb)
#pragma unroll
          for (int rr = (rb == 0 ? 1 : 0); rr < 16; rr += 2)
            red = (rr + 1 < 16) ? fmin3(red, s[rb][rr], s[rb][rr + 1]) : __builtin_fminf(red, s[rb][rr]);
        red = __builtin_fminf(red, xor32(red));
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
      const float nm = -m_run;
      bf16x8 pb[BK / 16];
      float lsum = 0.f;
#pragma unroll
      for (int rb = 0; rb < BK / 32; ++rb) {
        float p[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          float e = fast_exp2(__builtin_fmaf(s[rb][rr], cexp, nm));
          if (need_mask) e = ((vis[rb] >> rr) & 1u) ? e : 0.f;
          p[rr] = e;
          lsum += e;
        }
        pb[2 * rb] = pack8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
        pb[2 * rb + 1] = pack8(p[8], p[9], p[10], p[11], p[12], p[13], p[14], p[15]);
      }
      l_run += lsum;
      // O^T += V^T P^T
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const uint16_t *vr = vt + (32 * db + ql) * C::VS + 8 * hh;
#pragma unroll
        for (int kb = 0; kb < BK / 16; ++kb)
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ld16(vr + 16 * kb)), pb[kb], o[db], 0, 0, 0);
      }
    }
    if (j + 1 < nt) store_tile((j + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: out = O / l, lse = m ln2 + ln l -------------------------
  const float lt = l_run + xor32(l_run);
  if (qrow < a.Lq && kend_w > 0) {
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
  }
}

template <int D, int BK>
static hipError_t launch_t(const PrefillArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((prefill_kernel<D, BK>), dim3(a.total), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs &a, int D, hipStream_t s) {
  switch (D) {
    case 64: return launch_t<64, 64>(a, s);
    case 128: return launch_t<128, 64>(a, s);
    case 256: return launch_t<256, 32>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
