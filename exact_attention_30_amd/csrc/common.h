// Shared device helpers for the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

#define ATTN_DEV __device__ __forceinline__

// log2(e) in fp32: exp(x) = exp2(x * log2(e)); ln(2) for the way back.
#define ATTN_LOG2E 1.4426950408889634f
#define ATTN_LN2 0.6931471805599453f

// A row's running maximum is only raised when a tile's maximum exceeds it by
// more than this many powers of two; until then the exponentials may reach
// 2^ATTN_RESCALE_SLACK, which fp32 sums and bf16 weights hold without loss of
// relative precision.  The final normalisation uses the same reference, so the
// result is unchanged (up to rounding).
#define ATTN_RESCALE_SLACK 8.0f

ATTN_DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Lane-pair exchange across the two halves of a wave64 (lane l <-> l ^ 32).
ATTN_DEV float xor32(float x) { return __shfl_xor(x, 32); }
ATTN_DEV float xor16(float x) { return __shfl_xor(x, 16); }

ATTN_DEV bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }
// Workgroup barrier that leaves direct global->LDS loads in flight.  A fenced
// barrier (__syncthreads) waits for every outstanding load of the wave,
// including those of tiles staged further ahead; here the caller first waits
// (s_waitcnt vmcnt(n)) for the loads whose data other waves read after the
// barrier.  This wave's own LDS reads and writes complete before it
// (lgkmcnt(0)), and the "memory" clobber keeps the compiler from moving any
// memory access across it.
ATTN_DEV void barrier_keep_loads() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), other counters left alone
  asm volatile("s_barrier" ::: "memory");
}

// A condition that is the same in every lane of the wave (computed from
// per-wave values the compiler cannot prove uniform), as a scalar value: a
// branch on it is a scalar branch, and the code it guards is skipped, not
// executed under an exec mask.
ATTN_DEV bool uniform(bool p) { return __builtin_amdgcn_readfirstlane(p ? 1 : 0) != 0; }

// 16-byte global load / store helpers.
ATTN_DEV u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
// Streaming load (nontemporal hint): for data read once, such as a KV cache
// during decode, so that it does not displace reusable lines from the caches.
ATTN_DEV u32x4 ld16_stream(const void *p) { return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p)); }
ATTN_DEV void st16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }

ATTN_DEV bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

ATTN_DEV bf16x8 pack8(float a0, float a1, float a2, float a3, float a4, float a5, float a6, float a7) {
  bf16x8 r;
  r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
  r[4] = (__bf16)a4; r[5] = (__bf16)a5; r[6] = (__bf16)a6; r[7] = (__bf16)a7;
  return r;
}

ATTN_DEV float fmax3(float a, float b, float c) { return __builtin_fmaxf(a, __builtin_fmaxf(b, c)); }
ATTN_DEV float fmin3(float a, float b, float c) { return __builtin_fminf(a, __builtin_fminf(b, c)); }

// Row reductions across the two halves of a wave64 (lane l with lane l ^ 32):
// v_permlane32_swap(v, v) returns {v[l], v[l ^ 32]} as a pair in every lane.
ATTN_DEV float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
ATTN_DEV float pair_min(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fminf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
ATTN_DEV float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}


// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane
// 4r + c supplies the address of 4 consecutive bf16 of row r; lane i receives
// element i % 4 of the chunk of lane 4r + i / 4 for r = 0..3, i.e. column i of
// the 4 x 16 block.
ATTN_DEV bf16x4 lds_tr16(const uint16_t *p) {
  // an address-space cast (not a round trip through an integer) keeps the
  // pointer's provenance, so the compiler can tell which LDS array is read
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4 *)(const_cast<uint16_t *>(p)));
  return __builtin_bit_cast(bf16x4, r);
}

// Address spaces of the direct global -> LDS loads (global_load_lds_dwordx4).
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// Raw buffer resource over `bytes` bytes from `base` (no stride, the
// descriptor word of the gfx9 family): loads at offsets at or past `bytes`
// return zeros instead of reading memory.  The resource type exists only in
// the device compilation pass; kernel code that uses it is compiled under
// ATTN_DEVICE_PASS (the host pass only needs the kernels' signatures).
#if defined(__HIP_DEVICE_COMPILE__)
#define ATTN_DEVICE_PASS 1
ATTN_DEV __amdgpu_buffer_rsrc_t buf_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
// The same for a base and size that are uniform across the wave but that the
// compiler may not prove so (they are moved to scalar registers, so the loads
// take them as an operand directly).
ATTN_DEV __amdgpu_buffer_rsrc_t buf_rsrc_uniform(const void *base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p), hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  return buf_rsrc(reinterpret_cast<const void *>(((uint64_t)hi << 32) | lo), __builtin_amdgcn_readfirstlane(bytes));
}
#else
#define ATTN_DEVICE_PASS 0
#endif

// LDS row swizzles.  A tile row is stored unpadded; its 16-byte chunk c sits
// at chunk c ^ swz(row).  K: the b128 operand reads (16 rows, one chunk) then
// hit 16 distinct bank groups.  V: the swizzle moves whole 64-byte groups, so
// each transposing read still finds its 4 chunks together, and 4 consecutive
// rows land in 4 distinct bank quarters.
template <int D>
ATTN_DEV int kswz(int r) { return D == 64 ? ((r >> 1) & 7) : (r & 15); }
template <int D>
ATTN_DEV int vswz(int r) { return D == 64 ? 4 * ((r >> 1) & 1) : 4 * (r & 3); }
