// The C ABI of libattn.so: argument checks, launch shapes, workspace.
// The public contract (types, layouts, ownership, errors) is in include/attn.h.
#include <math.h>
#include <mutex>

#include "../../include/attn.h"
#include "kernels.h"

using attn::DecodeArgs;
using attn::PrefillArgs;

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

int decode_split_auto(int B, int Hkv, int Lmax) {
  // Aim for about 16K chunk-workgroups over the allocated cache extent (the
  // lengths are on the device), in powers of two between 256 and 1024 keys.
  const double work = (double)B * Hkv * Lmax;
  int s = 1024;
  while (s > 256 && work / s < 16384.0) s >>= 1;
  return s;
}

struct DecodeShape {
  int split, nsplit;
  size_t part_o_bytes, part_lse_bytes, total;
};

int decode_shape(int B, int Hq, int Hkv, int Lmax, int D, int split_keys, DecodeShape *ds) {
  if (split_keys != 0 && (split_keys < 0 || split_keys % 128 != 0)) return ATTN_ERR_SPLIT;
  const int split = split_keys ? split_keys : decode_split_auto(B, Hkv, Lmax);
  const int nsplit = (int)(((long long)Lmax + split - 1) / split);
  ds->split = split;
  ds->nsplit = nsplit;
  if (nsplit <= 1) {
    ds->part_o_bytes = ds->part_lse_bytes = ds->total = 0;
    return ATTN_OK;
  }
  const size_t rows = (size_t)B * Hq * nsplit;
  ds->part_o_bytes = (rows * D * sizeof(float) + 255) & ~(size_t)255;
  ds->part_lse_bytes = (rows * sizeof(float) + 255) & ~(size_t)255;
  ds->total = ds->part_o_bytes + ds->part_lse_bytes;
  return ATTN_OK;
}

int decode_check(const void *q, const void *kc, const void *vc, const int32_t *lens, const void *out, int B,
                 int Hq, int Hkv, int Lmax, int D, float scale) {
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ATTN_ERR_GQA;
  if (!head_dim_ok(D)) return ATTN_ERR_HEADDIM;
  if (!isfinite(scale)) return ATTN_ERR_SCALE;
  if (B < 0 || Lmax < 1 || B > 65535) return ATTN_ERR_SHAPE;
  if (B > 0 && (!q || !kc || !vc || !lens || !out)) return ATTN_ERR_NULL;
  const int n_hg = (Hq / Hkv + 63) / 64;
  if ((long long)Hkv * n_hg > 65535) return ATTN_ERR_SHAPE;
  // element counts must fit comfortably in 64-bit offsets
  if ((double)B * Hkv * (double)Lmax * D > 9.0e18) return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

int run_decode(const void *q, const void *kc, const void *vc, const int32_t *lens, void *out, float *lse, int B,
               int Hq, int Hkv, int Lmax, int D, float scale, int split_keys, void *ws, size_t ws_bytes,
               void *stream) {
  int st = decode_check(q, kc, vc, lens, out, B, Hq, Hkv, Lmax, D, scale);
  if (st != ATTN_OK) return st;
  DecodeShape ds;
  st = decode_shape(B, Hq, Hkv, Lmax, D, split_keys, &ds);
  if (st != ATTN_OK) return st;
  if (ws != nullptr && ws_bytes < ds.total) return ATTN_ERR_WORKSPACE;
  if (B == 0) return ATTN_OK;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void *mem = ws;
  bool owned = false;
  if (ds.total > 0 && mem == nullptr) {
    hipMemPool_t pool;
    if (device_pool(&pool) != hipSuccess) return ATTN_ERR_HIP;
    if (hipMallocFromPoolAsync(&mem, ds.total, pool, s) != hipSuccess) return ATTN_ERR_HIP;
    owned = true;
  }
  DecodeArgs a;
  a.q = static_cast<const uint16_t *>(q);
  a.kc = static_cast<const uint16_t *>(kc);
  a.vc = static_cast<const uint16_t *>(vc);
  a.lens = lens;
  a.out = static_cast<uint16_t *>(out);
  a.lse = lse;
  a.part_o = ds.total ? static_cast<float *>(mem) : nullptr;
  a.part_lse = ds.total ? reinterpret_cast<float *>(static_cast<char *>(mem) + ds.part_o_bytes) : nullptr;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Lmax = Lmax;
  a.G = Hq / Hkv;
  a.n_hg = (a.G + 63) / 64;
  a.split = ds.split;
  a.nsplit = ds.nsplit;
  a.c = scale * kLog2e;
  hipError_t e = attn::launch_decode(a, D, s);
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
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ATTN_ERR_GQA;
  if (!head_dim_ok(D)) return ATTN_ERR_HEADDIM;
  if (!isfinite(scale)) return ATTN_ERR_SCALE;
  if (B < 0 || Lq < 0 || Lk < 0) return ATTN_ERR_SHAPE;
  if (B == 0 || Lq == 0) return ATTN_OK;  // empty: nothing read or written, pointers may be NULL
  if (!q || !k || !v || !out) return ATTN_ERR_NULL;
  if (Lk == 0) return ATTN_ERR_SHAPE;
  if (causal && Lq > Lk) return ATTN_ERR_SHAPE;
  if ((double)B * Hq * (double)Lq * D > 9.0e18 || (double)B * Hkv * (double)Lk * D > 9.0e18) return ATTN_ERR_SHAPE;

  PrefillArgs a;
  a.q = static_cast<const uint16_t *>(q);
  a.k = static_cast<const uint16_t *>(k);
  a.v = static_cast<const uint16_t *>(v);
  a.out = static_cast<uint16_t *>(out);
  a.lse = lse;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Lq = Lq;
  a.Lk = Lk;
  a.G = Hq / Hkv;
  if (!attn::prefill_plan(a, D)) return ATTN_ERR_SHAPE;
  a.causal = causal ? 1 : 0;
  a.c = scale * kLog2e;
  hipError_t e = attn::launch_prefill(a, D, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_decode(const void *q, const void *kcache, const void *vcache, const int32_t *kv_lens, void *out, int B,
                int Hq, int Hkv, int Lmax, int D, float scale, void *stream) {
  return run_decode(q, kcache, vcache, kv_lens, out, nullptr, B, Hq, Hkv, Lmax, D, scale, 0, nullptr, 0, stream);
}

int attn_decode_ex(const void *q, const void *kcache, const void *vcache, const int32_t *kv_lens, void *out,
                   float *lse, int B, int Hq, int Hkv, int Lmax, int D, float scale, int split_keys,
                   void *workspace, size_t workspace_bytes, void *stream) {
  return run_decode(q, kcache, vcache, kv_lens, out, lse, B, Hq, Hkv, Lmax, D, scale, split_keys, workspace,
                    workspace_bytes, stream);
}

size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int Lmax, int D, int split_keys) {
  if (B <= 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || !head_dim_ok(D) || Lmax < 1) return 0;
  DecodeShape ds;
  if (decode_shape(B, Hq, Hkv, Lmax, D, split_keys, &ds) != ATTN_OK) return 0;
  return ds.total;
}

int attn_decode_split_keys(int B, int Hkv, int Lmax) {
  if (B < 1 || Hkv < 1 || Lmax < 1) return 0;
  return decode_split_auto(B, Hkv, Lmax);
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
    case ATTN_ERR_WORKSPACE: return "workspace smaller than attn_decode_workspace_bytes()";
    default: return "unknown status";
  }
}

}  // extern "C"
