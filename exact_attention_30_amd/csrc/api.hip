// The C ABI of libattn.so: argument checks, launch shapes, workspace.
// The public contract (types, layouts, ownership, errors) is in include/attn.h.
#include <math.h>
#include <mutex>

#include "../../include/attn.h"
#include "kernels.h"

using attn::DecodeArgs;
using attn::PrefillArgs;
using attn::BackwardArgs;

namespace {

constexpr float kLog2e = 1.4426950408889634f;

bool head_dim_ok(int D) { return D == 64 || D == 128 || D == 256; }

// The memory pool attn_decode takes its partials from: one per device, kept
// (release threshold at its maximum) so that repeated calls reuse memory.
std::mutex g_pool_mu;
hipMemPool_t g_pools[64];
bool g_pool_init[64];

hipError_t device_pool(hipMemPool_t *pool) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_pool_mu);
  if (!g_pool_init[dev]) {
    hipMemPoolProps props = {};
    props.allocType = hipMemAllocationTypePinned;
    props.handleTypes = hipMemHandleTypeNone;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    e = hipMemPoolCreate(&g_pools[dev], &props);
    if (e != hipSuccess) return e;
    uint64_t thr = UINT64_MAX;
    e = hipMemPoolSetAttribute(g_pools[dev], hipMemPoolAttrReleaseThreshold, &thr);
    if (e != hipSuccess) return e;
    g_pool_init[dev] = true;
  }
  *pool = g_pools[dev];
  return hipSuccess;
}

struct DecodeShape {
  int waves;        // main-kernel waves (ranges of the flat key-block space)
  size_t pre_bytes, part_lse_bytes, part_o_bytes, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace layout: pre [B + 1] int64 | part_lse [slots][GW] | part_o [slots][GW][D],
// slots = wave_slots + B * Hkv * n_hg, with wave_slots = kDecodeMaxWaves for a
// size independent of the device; a KV head has G * T query rows, in groups
// of up to decode_group(D) (GW = the group size).
void decode_workspace(int B, int Hq, int Hkv, int T, int D, DecodeShape *ds,
                      long long wave_slots = attn::kDecodeMaxWaves) {
  const long long GT = (long long)(Hq / Hkv) * T;
  const int grp = attn::decode_group(D);
  const long long hh = (long long)Hkv * ((GT + grp - 1) / grp);
  const long long gw = GT < grp ? GT : grp;
  const size_t slots = (size_t)wave_slots + (size_t)B * hh;
  ds->pre_bytes = align256((size_t)(B + 1) * sizeof(long long));
  ds->part_lse_bytes = align256(slots * gw * sizeof(float));
  ds->part_o_bytes = align256(slots * gw * D * sizeof(float));
  ds->total = ds->pre_bytes + ds->part_lse_bytes + ds->part_o_bytes;
}

// Waves of the main kernel: all resident wave slots of the device by default;
// with split_keys, enough waves that no wave gets more than split_keys keys
// when every sequence has Lmax keys (capped at kDecodeMaxWaves).
std::mutex g_occ_mu;
int g_occ_cache[64][3][3][2][2];

// 32-key blocks of a decode, bounded from the shapes: every sequence at Lmax
// keys (with a window, the keys its rows can see)
long long decode_block_bound(int B, int Hkv, int GT, int T, int window, int Lmax, int D) {
  const long long n_hg = (GT + attn::decode_group(D) - 1) / attn::decode_group(D);
  long long keys = Lmax;
  if (window > 0 && (long long)window + T + 31 < keys) keys = (long long)window + T + 31;
  return (long long)B * Hkv * n_hg * ((keys + 31) / 32);
}

// Whether a decode takes the wide-group kernel: kernel 0 chooses by the
// block bound, 1 never, 2 always (the caller has checked that the shape
// allows it).
bool decode_pick_wide(int D, int GT, bool q8, int B, int Hkv, int T, int window, int Lmax, int kernel = 0) {
  if (kernel == 1) return false;
  if (kernel == 2) return true;
  return attn::decode_use_wide(D, GT, q8, decode_block_bound(B, Hkv, GT, T, window, Lmax, D));
}

int device_waves(int D, int GT, bool q8, bool wide, int *waves) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return ATTN_ERR_HIP;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return ATTN_ERR_HIP;
  const int gw = GT < attn::decode_group(D) ? GT : attn::decode_group(D);
  const int ci = (gw + 15) / 16 >= 3 ? 2 : (gw + 15) / 16 - 1;
  const int di = D == 64 ? 0 : (D == 128 ? 1 : 2);
  std::lock_guard<std::mutex> lk(g_occ_mu);
  int &occ = g_occ_cache[dev][di][ci][q8 ? 1 : 0][wide ? 1 : 0];
  if (occ == 0 && attn::decode_waves_per_cu(D, gw, q8, wide, &occ) != hipSuccess) return ATTN_ERR_HIP;
  const long long w = (long long)cus * (occ > 0 ? occ : 1);
  *waves = (int)(w < attn::kDecodeMaxWaves ? w : attn::kDecodeMaxWaves);
  return ATTN_OK;
}

int decode_waves(int B, int Hq, int Hkv, int T, int Lmax, int D, int split_keys, bool q8, bool wide, int *waves) {
  const int GT = (Hq / Hkv) * T;
  if (split_keys == 0) return device_waves(D, GT, q8, wide, waves);
  const double keys = (double)B * Hkv * ((GT + attn::decode_group(D) - 1) / attn::decode_group(D)) *
                      (double)((Lmax + 31) / 32) * 32.0;
  double w = keys / split_keys;
  if (w < 1) w = 1;
  if (w > attn::kDecodeMaxWaves) w = attn::kDecodeMaxWaves;
  *waves = (int)w;
  if (*waves < w) ++*waves;
  if (*waves > attn::kDecodeMaxWaves) *waves = attn::kDecodeMaxWaves;
  return ATTN_OK;
}

int decode_check(const void *q, const void *kc, const void *vc, const int32_t *lens, const void *out, int B,
                 int Hq, int Hkv, int T, int Lmax, int D, float scale) {
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ATTN_ERR_GQA;
  if (!head_dim_ok(D)) return ATTN_ERR_HEADDIM;
  if (!isfinite(scale)) return ATTN_ERR_SCALE;
  if (B < 0 || Lmax < 1 || B > 65535 || T < 1 || T > Lmax) return ATTN_ERR_SHAPE;
  if (B > 0 && (!q || !kc || !vc || !lens || !out)) return ATTN_ERR_NULL;
  if ((long long)B * Hq * T > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  // element counts must fit comfortably in 64-bit offsets
  if ((double)B * Hkv * (double)Lmax * D > 9.0e18) return ATTN_ERR_SHAPE;
  // one sequence's cache rows of one KV head are read through a buffer
  // resource with 32-bit offsets: at most 2^31 - 1 bytes (2 GiB)
  if ((long long)Lmax * D * 2 >= (1LL << 31)) return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

// Static scratch of attn_decode_noalloc: the decode's partials for callers
// that cannot allocate.  The array is a file-scope device variable, so every
// device holds its own copy (at its own address) from the library's load on
// that device until the process ends.  Host code never uses the array's name
// as an address: the address is looked up per device (scratch_address).
constexpr size_t kScratchBytes = (size_t)64 << 20;
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void *g_scratch[64];

// The device address of `scratch` on the current device (looked up once per
// device, with that device current).
int scratch_address(void **ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return ATTN_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return ATTN_ERR_HIP;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return ATTN_OK;
}

// kscale / vscale: per-block fp16 scales of int8 caches (both null for bf16
// caches; q8 says which the caller meant, so a missing scale is an error).
// kernel: 0 automatic, 1 decode_main_kernel, 2 decode_wide_kernel (must be
// able to serve the shape, else ATTN_ERR_KERNEL).
// use_scratch: the partials go to the static scratch, laid out for the actual
// wave count; sizes that need more than kScratchBytes are ATTN_ERR_SCRATCH,
// and nothing is allocated.
int run_decode(const void *q, const void *kc, const void *vc, const int32_t *lens, void *out, float *lse, int B,
               int Hq, int Hkv, int T, int window, int Lmax, int D, float scale, int split_keys, void *ws,
               size_t ws_bytes, void *stream, bool q8 = false, const void *kscale = nullptr,
               const void *vscale = nullptr, int kernel = 0, bool use_scratch = false) {
  int st = decode_check(q, kc, vc, lens, out, B, Hq, Hkv, T, Lmax, D, scale);
  if (st != ATTN_OK) return st;
  if (q8 && B > 0 && (kscale == nullptr || vscale == nullptr)) return ATTN_ERR_NULL;
  if (window < 0) return ATTN_ERR_SHAPE;
  if (split_keys != 0 && (split_keys < 0 || split_keys % 128 != 0)) return ATTN_ERR_SPLIT;
  if (kernel < 0 || kernel > 2) return ATTN_ERR_KERNEL;
  if (kernel == 2 && !attn::decode_use_wide(D, (Hq / Hkv) * T, q8, attn::kDecodeWideMinBlocks))
    return ATTN_ERR_KERNEL;
  DecodeShape ds;
  decode_workspace(B, Hq, Hkv, T, D, &ds);
  if (ws != nullptr && ws_bytes < ds.total) return ATTN_ERR_WORKSPACE;
  if (B == 0) return ATTN_OK;
  const bool wide =
      decode_pick_wide(D, (Hq / Hkv) * T, q8, B, Hkv, T, window < Lmax ? window : 0, Lmax, kernel);
  st = decode_waves(B, Hq, Hkv, T, Lmax, D, split_keys, q8, wide, &ds.waves);
  if (st != ATTN_OK) return st;
  if (use_scratch) {
    const int waves = ds.waves;
    decode_workspace(B, Hq, Hkv, T, D, &ds, waves);
    ds.waves = waves;
    if (ds.total > kScratchBytes) return ATTN_ERR_SCRATCH;
    st = scratch_address(&ws);
    if (st != ATTN_OK) return st;
  }

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void *mem = ws;
  bool owned = false;
  if (mem == nullptr) {
    hipMemPool_t pool;
    if (device_pool(&pool) != hipSuccess) return ATTN_ERR_HIP;
    if (hipMallocFromPoolAsync(&mem, ds.total, pool, s) != hipSuccess) return ATTN_ERR_HIP;
    owned = true;
  }
  char *base = static_cast<char *>(mem);
  DecodeArgs a;
  a.q = static_cast<const uint16_t *>(q);
  a.kc = static_cast<const uint16_t *>(kc);
  a.vc = static_cast<const uint16_t *>(vc);
  a.lens = lens;
  a.out = static_cast<uint16_t *>(out);
  a.lse = lse;
  a.kscale = q8 ? static_cast<const uint16_t *>(kscale) : nullptr;
  a.vscale = q8 ? static_cast<const uint16_t *>(vscale) : nullptr;
  a.pre = reinterpret_cast<long long *>(base);
  a.part_lse = reinterpret_cast<float *>(base + ds.pre_bytes);
  a.part_o = reinterpret_cast<float *>(base + ds.pre_bytes + ds.part_lse_bytes);
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Lmax = Lmax;
  a.G = Hq / Hkv;
  a.T = T;
  a.window = window < Lmax ? window : 0;   // a window of Lmax or more keys hides nothing
  a.n_hg = (a.G * T + attn::decode_group(D) - 1) / attn::decode_group(D);
  a.c = scale * kLog2e;
  a.wide = wide ? 1 : 0;
  hipError_t e = attn::launch_decode(a, D, ds.waves, s);
  if (owned) {
    hipError_t f = hipFreeAsync(mem, s);
    if (e == hipSuccess) e = f;
  }
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int device_cus(int *cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ATTN_ERR_HIP;
  if (hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return ATTN_ERR_HIP;
  if (*cus < 1) *cus = 1;
  return ATTN_OK;
}

// Argument checks and launch shape of a prefill (everything but pointers).
// splits: 0 chooses the key-split count: 1 when the grid already has at least
// two workgroups per compute unit, else enough ranges for that (each of at
// least 8 tiles, at most 32 ranges); otherwise 1..kPrefillMaxSplits.
int prefill_setup(PrefillArgs *pa, int B, int Hq, int Hkv, int Lq, int Lk, int D, int causal, int window,
                  float scale, int splits) {
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ATTN_ERR_GQA;
  if (!head_dim_ok(D)) return ATTN_ERR_HEADDIM;
  if (!isfinite(scale)) return ATTN_ERR_SCALE;
  if (B < 0 || Lq < 0 || Lk < 0 || window < 0 || (window > 0 && !causal)) return ATTN_ERR_SHAPE;
  if (splits < 0 || splits > attn::kPrefillMaxSplits) return ATTN_ERR_SPLIT;
  if (B == 0 || Lq == 0) {
    pa->nsplit = 0;
    return ATTN_OK;
  }
  if (Lk == 0) return ATTN_ERR_SHAPE;
  if (causal && Lq > Lk) return ATTN_ERR_SHAPE;
  if ((double)B * Hq * (double)Lq * D > 9.0e18 || (double)B * Hkv * (double)Lk * D > 9.0e18) return ATTN_ERR_SHAPE;
  PrefillArgs &a = *pa;
  a = PrefillArgs{};
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Lq = Lq;
  a.Lk = Lk;
  a.G = Hq / Hkv;
  a.causal = causal ? 1 : 0;
  a.window = (causal && window < Lk) ? window : 0;   // a window of Lk or more keys hides nothing
  a.c = scale * kLog2e;
  a.nsplit = 1;
  if (!attn::prefill_plan(a, D)) return ATTN_ERR_SHAPE;
  int ns = splits;
  if (ns == 0) {
    // Small grids: cut each query block's keys into ns ranges.  With S
    // resident workgroups on the device, u workgroups of work w take
    // ceil(u ns / S) rounds of w / ns each; every range adds a partial
    // output to merge (a small cost per range).  Pick the cheapest ns.
    int cus = 0, occ = 0;
    if (device_cus(&cus) != ATTN_OK) return ATTN_ERR_HIP;
    if (attn::prefill_wgs_per_cu(D, &occ) != hipSuccess) return ATTN_ERR_HIP;
    const long long slots = (long long)cus * (occ > 0 ? occ : 1);
    const long long units = a.total;
    ns = 1;
    if (units < 2 * slots) {
      const int tk = attn::prefill_tile_keys(D);
      const long long keys = a.window ? (long long)a.window + a.Bq : (long long)Lk;   // per query block, at most
      long long cap = (keys + tk - 1) / tk / 8;
      if (cap > 32) cap = 32;
      double best = (double)((units + slots - 1) / slots);
      for (long long n = 2; n <= cap; ++n) {
        const double cost = (double)((units * n + slots - 1) / slots) / n + 0.02 * n;
        if (cost < best - 1e-9) {
          best = cost;
          ns = (int)n;
        }
      }
    }
  }
  a.nsplit = ns;
  if (!attn::prefill_plan(a, D)) return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

// Workspace of a split prefill: part_lse [rows][nsplit] | part_o [rows][nsplit][D].
size_t prefill_lse_bytes(const PrefillArgs &a) {
  return align256((size_t)a.B * a.Hq * (size_t)a.Lq * a.nsplit * sizeof(float));
}
size_t prefill_workspace(const PrefillArgs &a, int D) {
  if (a.nsplit <= 1) return 0;
  return prefill_lse_bytes(a) + align256((size_t)a.B * a.Hq * (size_t)a.Lq * a.nsplit * D * sizeof(float));
}

int run_prefill(const void *q, const void *k, const void *v, void *out, float *lse, int B, int Hq, int Hkv, int Lq,
                int Lk, int D, int causal, int window, float scale, int splits, void *ws, size_t ws_bytes,
                void *stream) {
  // checks in the documented order; prefill_setup repeats the first ones
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ATTN_ERR_GQA;
  if (!head_dim_ok(D)) return ATTN_ERR_HEADDIM;
  if (!isfinite(scale)) return ATTN_ERR_SCALE;
  if (B < 0 || Lq < 0 || Lk < 0 || window < 0 || (window > 0 && !causal)) return ATTN_ERR_SHAPE;
  if (splits < 0 || splits > attn::kPrefillMaxSplits) return ATTN_ERR_SPLIT;
  if (B == 0 || Lq == 0) return ATTN_OK;  // empty: nothing read or written, pointers may be NULL
  if (!q || !k || !v || !out) return ATTN_ERR_NULL;
  PrefillArgs a;
  int st = prefill_setup(&a, B, Hq, Hkv, Lq, Lk, D, causal, window, scale, splits);
  if (st != ATTN_OK) return st;
  const size_t need = prefill_workspace(a, D);
  if (ws != nullptr && ws_bytes < need) return ATTN_ERR_WORKSPACE;
  a.q = static_cast<const uint16_t *>(q);
  a.k = static_cast<const uint16_t *>(k);
  a.v = static_cast<const uint16_t *>(v);
  a.out = static_cast<uint16_t *>(out);
  a.lse = lse;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void *mem = ws;
  bool owned = false;
  if (need > 0 && mem == nullptr) {
    hipMemPool_t pool;
    if (device_pool(&pool) != hipSuccess) return ATTN_ERR_HIP;
    if (hipMallocFromPoolAsync(&mem, need, pool, s) != hipSuccess) return ATTN_ERR_HIP;
    owned = true;
  }
  if (need > 0) {
    char *base = static_cast<char *>(mem);
    a.part_lse = reinterpret_cast<float *>(base);
    a.part_o = reinterpret_cast<float *>(base + prefill_lse_bytes(a));
  }
  if (a.nsplit == 1 && attn::prefill_can_persist(D)) {
    // large grids: one resident workgroup per slot, several work items each
    int cus = 0, occ = 0;
    if (device_cus(&cus) != ATTN_OK) return ATTN_ERR_HIP;
    if (attn::prefill_wgs_per_cu(D, &occ) != hipSuccess) return ATTN_ERR_HIP;
    const long long slots = (long long)cus * (occ > 0 ? occ : 1);
    if (slots % 8 == 0 && (long long)a.total >= 2 * slots) a.persist = (int)slots;
  }
  hipError_t e = attn::launch_prefill(a, D, s);
  if (owned) {
    hipError_t f = hipFreeAsync(mem, s);
    if (e == hipSuccess) e = f;
  }
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // namespace

extern "C" {

int attn_prefill(const void *q, const void *k, const void *v, void *out, float *lse, int B, int Hq, int Hkv,
                 int Lq, int Lk, int D, int causal, float scale, void *stream) {
  return run_prefill(q, k, v, out, lse, B, Hq, Hkv, Lq, Lk, D, causal, 0, scale, 0, nullptr, 0, stream);
}

int attn_prefill_ex(const void *q, const void *k, const void *v, void *out, float *lse, int B, int Hq, int Hkv,
                    int Lq, int Lk, int D, int causal, int window, float scale, int splits, void *workspace,
                    size_t workspace_bytes, void *stream) {
  return run_prefill(q, k, v, out, lse, B, Hq, Hkv, Lq, Lk, D, causal, window, scale, splits, workspace,
                     workspace_bytes, stream);
}

int attn_prefill_splits(int B, int Hq, int Hkv, int Lq, int Lk, int D, int causal, int window, int splits) {
  PrefillArgs a;
  int st = prefill_setup(&a, B, Hq, Hkv, Lq, Lk, D, causal, window, 1.f, splits);
  return st == ATTN_OK ? a.nsplit : 0;
}

size_t attn_prefill_workspace_bytes(int B, int Hq, int Hkv, int Lq, int Lk, int D, int causal, int window,
                                    int splits) {
  PrefillArgs a;
  if (prefill_setup(&a, B, Hq, Hkv, Lq, Lk, D, causal, window, 1.f, splits) != ATTN_OK) return 0;
  return prefill_workspace(a, D);
}

size_t attn_backward_workspace_bytes(int B, int Hq, int Lq) {
  if (B <= 0 || Hq < 1 || Lq <= 0) return 0;
  return 2 * align256((size_t)B * Hq * Lq * sizeof(float));
}

int attn_backward(const void *q, const void *k, const void *v, const void *out, const void *dout, const float *lse,
                  void *dq, void *dk, void *dv, int B, int Hq, int Hkv, int Lq, int Lk, int D, int causal, int window,
                  float scale, void *workspace, size_t workspace_bytes, void *stream) {
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ATTN_ERR_GQA;
  if (!head_dim_ok(D)) return ATTN_ERR_HEADDIM;
  if (!isfinite(scale)) return ATTN_ERR_SCALE;
  if (B < 0 || Lq < 0 || Lk < 0 || window < 0 || (window > 0 && !causal)) return ATTN_ERR_SHAPE;
  if (B == 0 || (Lq == 0 && Lk == 0)) return ATTN_OK;
  if (Lk == 0 || Lq == 0) return ATTN_ERR_SHAPE;   // rows without keys, or keys without rows: no gradient defined
  if (causal && Lq > Lk) return ATTN_ERR_SHAPE;
  if ((double)B * Hq * (double)Lq * D > 9.0e18 || (double)B * Hkv * (double)Lk * D > 9.0e18) return ATTN_ERR_SHAPE;
  if ((long long)B * Hkv * ((Lk + 127) / 128) > 0x7fffffffLL || (long long)B * Hq * ((Lq + 31) / 32) > 0x7fffffffLL)
    return ATTN_ERR_SHAPE;
  if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv) return ATTN_ERR_NULL;
  const size_t need = attn_backward_workspace_bytes(B, Hq, Lq);
  if (workspace != nullptr && workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  BackwardArgs a;
  a.q = static_cast<const uint16_t *>(q);
  a.k = static_cast<const uint16_t *>(k);
  a.v = static_cast<const uint16_t *>(v);
  a.out = static_cast<const uint16_t *>(out);
  a.dout = static_cast<const uint16_t *>(dout);
  a.lse = lse;
  a.dq = static_cast<uint16_t *>(dq);
  a.dk = static_cast<uint16_t *>(dk);
  a.dv = static_cast<uint16_t *>(dv);
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Lq = Lq;
  a.Lk = Lk;
  a.G = Hq / Hkv;
  a.causal = causal ? 1 : 0;
  a.window = (causal && window < Lk) ? window : 0;
  a.dq_hpw = attn::backward_dq_heads(a.G);
  a.scale = scale;
  a.c = scale * kLog2e;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void *mem = workspace;
  bool owned = false;
  if (mem == nullptr) {
    hipMemPool_t pool;
    if (device_pool(&pool) != hipSuccess) return ATTN_ERR_HIP;
    if (hipMallocFromPoolAsync(&mem, need, pool, s) != hipSuccess) return ATTN_ERR_HIP;
    owned = true;
  }
  a.delta = static_cast<float *>(mem);
  a.lse2 = reinterpret_cast<float *>(static_cast<char *>(mem) + need / 2);
  hipError_t e = attn::launch_backward(a, D, s);
  if (owned) {
    hipError_t f = hipFreeAsync(mem, s);
    if (e == hipSuccess) e = f;
  }
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_decode(const void *q, const void *kcache, const void *vcache, const int32_t *kv_lens, void *out, int B,
                int Hq, int Hkv, int Lmax, int D, float scale, void *stream) {
  return run_decode(q, kcache, vcache, kv_lens, out, nullptr, B, Hq, Hkv, 1, 0, Lmax, D, scale, 0, nullptr, 0,
                    stream);
}

int attn_decode_noalloc(const void *q, const void *kcache, const void *vcache, const int32_t *kv_lens, void *out,
                        int B, int Hq, int Hkv, int Lmax, int D, float scale, void *stream) {
  return run_decode(q, kcache, vcache, kv_lens, out, nullptr, B, Hq, Hkv, 1, 0, Lmax, D, scale, 0, nullptr, 0, stream,
                    false, nullptr, nullptr, 0, true);
}

size_t attn_decode_noalloc_max_bytes(void) { return kScratchBytes; }

int attn_decode_ex(const void *q, const void *kcache, const void *vcache, const int32_t *kv_lens, void *out,
                   float *lse, int B, int Hq, int Hkv, int Lmax, int D, float scale, int split_keys, void *stream) {
  return run_decode(q, kcache, vcache, kv_lens, out, lse, B, Hq, Hkv, 1, 0, Lmax, D, scale, split_keys, nullptr, 0,
                    stream);
}

int attn_decode_multi(const void *q, const void *kcache, const void *vcache, const int32_t *kv_lens, void *out,
                      float *lse, int B, int Hq, int Hkv, int T, int window, int Lmax, int D, float scale,
                      void *workspace, size_t workspace_bytes, void *stream) {
  return run_decode(q, kcache, vcache, kv_lens, out, lse, B, Hq, Hkv, T, window, Lmax, D, scale, 0, workspace,
                    workspace_bytes, stream);
}

int attn_decode_multi_ex(const void *q, const void *kcache, const void *vcache, const int32_t *kv_lens, void *out,
                         float *lse, int B, int Hq, int Hkv, int T, int window, int Lmax, int D, float scale,
                         int split_keys, int kernel, void *workspace, size_t workspace_bytes, void *stream) {
  return run_decode(q, kcache, vcache, kv_lens, out, lse, B, Hq, Hkv, T, window, Lmax, D, scale, split_keys,
                    workspace, workspace_bytes, stream, false, nullptr, nullptr, kernel);
}

int attn_decode_q8(const void *q, const void *kq, const void *kscale, const void *vq, const void *vscale,
                   const int32_t *kv_lens, void *out, float *lse, int B, int Hq, int Hkv, int T, int window, int Lmax,
                   int D, float scale, void *workspace, size_t workspace_bytes, void *stream) {
  return run_decode(q, kq, vq, kv_lens, out, lse, B, Hq, Hkv, T, window, Lmax, D, scale, 0, workspace,
                    workspace_bytes, stream, true, kscale, vscale);
}

size_t attn_decode_multi_workspace_bytes(int B, int Hq, int Hkv, int T, int Lmax, int D) {
  if (B <= 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || !head_dim_ok(D) || Lmax < 1 || T < 1 || T > Lmax) return 0;
  DecodeShape ds;
  decode_workspace(B, Hq, Hkv, T, D, &ds);
  return ds.total;
}

int attn_decode_waves(int B, int Hq, int Hkv, int Lmax, int D, int split_keys) {
  if (B <= 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || !head_dim_ok(D) || Lmax < 1) return 0;
  if (split_keys != 0 && (split_keys < 0 || split_keys % 128 != 0)) return 0;
  int w = 0;
  const bool wide = decode_pick_wide(D, Hq / Hkv, false, B, Hkv, 1, 0, Lmax);
  return decode_waves(B, Hq, Hkv, 1, Lmax, D, split_keys, false, wide, &w) == ATTN_OK ? w : 0;
}

const char *attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "invalid sizes (negative, empty key set, causal with Lq > Lk, Lmax < 1, or too large)";
    case ATTN_ERR_HEADDIM: return "head dim must be 64, 128 or 256";
    case ATTN_ERR_GQA: return "Hq and Hkv must be positive with Hq a multiple of Hkv";
    case ATTN_ERR_SCALE: return "scale must be finite";
    case ATTN_ERR_HIP: return "a HIP call or kernel launch failed";
    case ATTN_ERR_SPLIT: return "split_keys must be 0 or a positive multiple of 128";
    case ATTN_ERR_WORKSPACE: return "workspace smaller than the matching *_workspace_bytes()";
    case ATTN_ERR_KERNEL: return "kernel choice not 0, 1 or 2, or the chosen kernel cannot serve this shape";
    case ATTN_ERR_SCRATCH: return "sizes need more partials than the static scratch of attn_decode_noalloc holds";
    default: return "unknown status";
  }
}

}  // extern "C"
