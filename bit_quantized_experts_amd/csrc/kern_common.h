// kern_common.h -- device helpers shared by the HIP kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_internal.h"

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#define DEVI __device__ __forceinline__

// The work-item index as a value the optimiser cannot see through.  Phase
// functions derive their per-lane addresses from it, so in a kernel that runs
// the phases in a loop (the persistent decode pass) those addresses are
// recomputed inside each phase instead of being hoisted out of the loop and
// kept live (or spilled) across every other phase.
DEVI int opaque_tid() {
  int t = (int)threadIdx.x;
  __asm__ volatile("" : "+v"(t));
  return t;
}

// ---------------------------------------------------------------------------
// Fragment decode.
//
// A fragment is 8 codes (one MFMA B operand of 16x16x32: inputs 8q..8q+7 of
// one weight row).  In the packed layout its codes sit in one nibble each of
// a dword after a mask: (w >> sh) & 0x33333333 leaves q (0..3) in the low two
// bits of every nibble.  A nibble 00qq read as an OCP fp4 (e2m1) value is
// q/2 (0, 0.5, 1, 1.5), so the gfx950 fp4->f16 conversion with scale 2.0 (a
// power of two: the conversion only uses the scale's exponent) yields q as an
// exact fp16 value; the byte select picks two codes at a time, low nibble to
// element 0.  The block offset 2^(b-1) and the fp16 block scale are applied
// outside (accumulator seed and epilogue), so nothing here rounds.
// ---------------------------------------------------------------------------
DEVI half8_t nibbles_to_half8(uint32_t D, float sc) {
  half2_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(D, sc, 0);
  half2_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(D, sc, 1);
  half2_t c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(D, sc, 2);
  half2_t d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(D, sc, 3);
  half8_t r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// q (unsigned code, 0..3) of fragment f from the lane's 4 code dwords.
DEVI half8_t frag_q2(const u32x4_t& w, int f) {
  uint32_t dw = w[f >> 1];
  uint32_t D = ((f & 1) ? (dw >> 2) : dw) & 0x33333333u;
  return nibbles_to_half8(D, 2.0f);
}

// q (unsigned code, 0..7) of fragment f for 3-bit codes: low two bits from
// the code dwords, high bit from the 2 high-bit dwords (fragment 4h+g at
// bit 4e+g of dword h); 000h read as fp4 is h/2, scale 8 gives 4h.
DEVI half8_t frag_q3(const u32x4_t& w, const u32x2_t& hbits, int f) {
  half8_t lo = frag_q2(w, f);
  uint32_t H = (hbits[f >> 2] >> (f & 3)) & 0x11111111u;
  half8_t hi = nibbles_to_half8(H, 8.0f);
  return lo + hi;
}

// ---------------------------------------------------------------------------
// The codebook grid of the layer being multiplied (codebook blocks only):
// 512 entries of 4 fp16 magnitudes, staged by load_grid at kernel start.
// Kernels of the b-bit kinds never touch it, so it takes no LDS there.
// ---------------------------------------------------------------------------
__shared__ uint2 cb_grid_lds[512];

// Stage the grid (all threads of the workgroup; a barrier must follow
// before the first fragment decode).  The block kinds are those of
// moe_launch.h: MOE_KIND_CB = 4.
template <int BITS>
DEVI void load_grid(const uint32_t* grid16, int tid, int nthreads) {
  if constexpr (BITS == 4)
    for (int i = tid; i < 512; i += nthreads) cb_grid_lds[i] = reinterpret_cast<const uint2*>(grid16)[i];
}

// ---------------------------------------------------------------------------
// Codebook fragments.  The lane's chunk data: 16 index bytes (bytes 2f and
// 2f+1: the low 8 bits of the two grid indices of fragment f, inputs 8q..8q+3
// and 8q+4..8q+7), 16 index high bits (bits 2f, 2f+1) and 64 sign bits (bits
// 8f..8f+7: inputs 8q..8q+7 of fragment f, set = negative).  The grid sits in
// LDS as 4 fp16 magnitudes per entry (two words), so one 64-bit LDS read
// gives 4 exact codes; the sign bits go into the fp16 sign bits by XOR.
// ---------------------------------------------------------------------------
DEVI half8_t frag_cb(const u32x4_t& idx, uint32_t hi, const u32x2_t& sg, int f, const uint2* grid) {
  const uint32_t w = idx[f >> 1] >> (16 * (f & 1));
  const uint32_t i0 = (w & 0xffu) | (((hi >> (2 * f)) & 1u) << 8);
  const uint32_t i1 = ((w >> 8) & 0xffu) | (((hi >> (2 * f + 1)) & 1u) << 8);
  const uint2 m0 = grid[i0], m1 = grid[i1];
  const uint32_t s = (sg[f >> 2] >> (8 * (f & 3))) & 0xffu;
  u32x4_t r;
  r[0] = m0.x ^ (((s & 1u) << 15) | ((s & 2u) << 30));
  r[1] = m0.y ^ (((s & 4u) << 13) | ((s & 8u) << 28));
  r[2] = m1.x ^ (((s & 16u) << 11) | ((s & 32u) << 26));
  r[3] = m1.y ^ (((s & 64u) << 9) | ((s & 128u) << 24));
  return __builtin_bit_cast(half8_t, r);
}

// ---------------------------------------------------------------------------
// Read-ahead: lines rank, rank + n, ... of the ranges in w (128-byte lines),
// one 4-byte load each into a 1 KB scratch LDS area (no registers, nothing
// written to memory), waited for before the workgroup's LDS is released.
// Every such load fetches its whole line into the memory-side cache.
// ---------------------------------------------------------------------------
template <typename WarmT>
DEVI void warm_lines(const WarmT& w, int rank, int n, void* lds_scratch) {
  typedef __attribute__((address_space(3))) void* lds_ptr_t;
  const int wv = threadIdx.x >> 6;
  char* sink = reinterpret_cast<char*>(lds_scratch) + 256 * (wv & 3);
  for (int r = 0; r < w.n; ++r) {
    const int64_t lines = w.bytes[r] >> 7;
    for (int64_t i = (int64_t)rank * blockDim.x + threadIdx.x; i < lines; i += (int64_t)n * blockDim.x)
      __builtin_amdgcn_global_load_lds(w.p[r] + 128 * i, (lds_ptr_t)sink, 4, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0);
}

// ---------------------------------------------------------------------------
// Buffer loads that bypass nothing special: plain 128/64-bit global loads.
// ---------------------------------------------------------------------------
DEVI u32x4_t ld128(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
DEVI u32x2_t ld64(const void* p) { return *reinterpret_cast<const u32x2_t*>(p); }
DEVI u32x4_t ld128_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
DEVI u32x2_t ld64_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
}

// ---------------------------------------------------------------------------
// Device-coherent accesses: values that workgroups hand to each other inside
// one kernel (or that another XCD's workgroup wrote) are stored and loaded
// with the sc1 cache policy, as agent-scope atomics are, so no XCD's L2 serves
// a stale copy and no cache write-back or invalidation is needed.  The
// 16-byte forms go through a raw buffer resource (offsets in bytes; an access
// past 2^31 - 1 bytes of the base reads zero instead of faulting).
// ---------------------------------------------------------------------------
DEVI void st_dev(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
DEVI float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEVI void st_dev_i(int32_t* p, int32_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
DEVI int32_t ld_dev_i(const int32_t* p) {
  return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEVI void st_dev_u(uint32_t* p, uint32_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
DEVI uint32_t ld_dev_u(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

DEVI __amdgpu_buffer_rsrc_t coh_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
}
constexpr int kCohSc1 = 16;  // cache-policy operand of the buffer intrinsics: sc1
DEVI float4_t coh_ld4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCohSc1));
}
DEVI u32x4_t coh_ld4u(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCohSc1));
}
DEVI void coh_st4(__amdgpu_buffer_rsrc_t r, uint32_t off, const float4_t& v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, off, 0, kCohSc1);
}

// Adds one to a counter other workgroups wait on (after the caller has made
// its own stores complete).
DEVI void signal_add(uint32_t* ctr, uint32_t n = 1u) {
  __hip_atomic_fetch_add(ctr, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroup-wide bounded wait until *ctr >= target: thread 0 polls, the
// others wait at the barrier.  Gives up (false in every thread) once the
// kernel's abort word is set by another workgroup, or after kSpinLimit polls
// (then it sets the abort word itself), so every wait ends and a pass whose
// workgroups cannot all make progress finishes early instead of hanging.
// `flag` is a workgroup-shared int.
constexpr uint32_t kSpinLimit = 1u << 21;
DEVI bool wg_wait(const uint32_t* ctr, uint32_t target, uint32_t* abort_w, int* flag) {
  if (threadIdx.x == 0) {
    int ok = 1;
    uint32_t n = 0;
    while (ld_dev_u(ctr) < target) {
      ++n;
      if ((n & 31u) == 0u && ld_dev_u(abort_w) != 0u) {
        ok = 0;
        break;
      }
      if (n > kSpinLimit) {
        st_dev_u(abort_w, 1u);
        ok = 0;
        break;
      }
      // a short pause between polls: many workgroups poll one line
      if (n < 8) __builtin_amdgcn_s_sleep(2);
      else __builtin_amdgcn_s_sleep(8);
    }
    *flag = ok;
  }
  __syncthreads();
  const bool ok = *flag != 0;
  __syncthreads();  // every thread has read the flag before it is reused
  return ok;
}

DEVI float half_bits_to_float(uint32_t h16) {
  _Float16 h;
  uint16_t b = (uint16_t)h16;
  __builtin_memcpy(&h, &b, 2);
  return (float)h;
}

DEVI float4_t mfma16x16x32(const half8_t& a, const half8_t& b, const float4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Swap halves: lanes 0..31 <-> 32..63; returns v + (value of the partner lane).
DEVI float add_partner32(float v) {
  uint32_t x = __float_as_uint(v);
  auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroup barrier that orders LDS accesses only: it waits for this wave's
// LDS operations, not for its global loads in flight (the fence of
// __syncthreads() waits for those too).
DEVI void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

DEVI float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

DEVI float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// ---------------------------------------------------------------------------
// Cross-lane moves that stay in the vector ALU (DPP and the gfx950 permlane
// swaps), for reductions whose operator is commutative: every step pairs
// each lane with a lane of the other half of a growing group, so after the
// six steps every lane holds the result over all 64 lanes.
//   quad_perm [1,0,3,2] and [2,3,0,1]: partners inside a group of 4 lanes,
//   row_half_mirror: lane i <-> 7-i inside 8, row_mirror: i <-> 15-i inside
//   16, permlane16 swap: row 0 <-> row 1 and row 2 <-> row 3, permlane32
//   swap: lanes 0..31 <-> 32..63.
// ---------------------------------------------------------------------------
DEVI uint32_t dpp_perm(uint32_t v, int step) {
  switch (step) {
    case 0: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);
    case 1: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);
    case 2: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, true);
    default: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, true);
  }
}

// Sum over the 4 lanes of a quad (lanes 4j..4j+3), in every lane of the quad.
DEVI float quad_sum(float v) {
  v += __uint_as_float(dpp_perm(__float_as_uint(v), 0));
  return v + __uint_as_float(dpp_perm(__float_as_uint(v), 1));
}

// Exponent e with 2^14 <= m * 2^-e < 2^15 (0 when m is 0 or not a number):
// scaling a vector by 2^-e (exact) puts its largest magnitude m at the top of
// the fp16 range, so an fp16 hi + lo split of it neither overflows nor loses
// its low part to subnormals.
DEVI int fp16_exponent_for(float m) {
  if (!(m > 0.f)) return 0;
  int e;
  frexpf(m, &e);  // m = f * 2^e, 0.5 <= f < 1
  return e - 15;
}

DEVI uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }
DEVI uint64_t u64_of(uint32_t lo, uint32_t hi) { return ((uint64_t)hi << 32) | lo; }

// Maximum of a 64-bit key over the wavefront, in every lane.
DEVI uint64_t wave_max_u64(uint64_t k) {
#pragma unroll
  for (int st = 0; st < 4; ++st) k = umax64(k, u64_of(dpp_perm((uint32_t)k, st), dpp_perm((uint32_t)(k >> 32), st)));
  {
    auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)k, (uint32_t)k, false, false);
    auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(k >> 32), (uint32_t)(k >> 32), false, false);
    k = umax64(u64_of(lo[0], hi[0]), u64_of(lo[1], hi[1]));
  }
  {
    auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)k, (uint32_t)k, false, false);
    auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(k >> 32), (uint32_t)(k >> 32), false, false);
    k = umax64(u64_of(lo[0], hi[0]), u64_of(lo[1], hi[1]));
  }
  return k;
}

// Sum over the 16 lanes of a row, in every lane of the row (fixed order).
DEVI float row16_sum(float v) {
#pragma unroll
  for (int st = 0; st < 4; ++st) v += __uint_as_float(dpp_perm(__float_as_uint(v), st));
  return v;
}

// ---------------------------------------------------------------------------
// Deterministic fp64 exponential for the gate weights.  Steps: n = rint(z /
// ln2); r = z - n*ln2 as two fused steps with ln2 split into a high part (the
// double nearest ln2) and a low part (the double nearest the remainder);
// p = sum_{i=0..13} r^i/i! by Horner with fused multiply-add, from i = 13
// down; result = p * 2^n.  Coefficients are 1/i! rounded once to double
// (i! <= 13! is exact in double, so 1.0 / i! is one correctly rounded
// division, done at compile time).  Any IEEE fp64 implementation of the same
// steps returns the same bits.
// ---------------------------------------------------------------------------
struct MoeExpCoeffs {
  double c[14];
};
// 1/i! for i = 0..13, evaluated at compile time: i! is built by exact
// multiplications (13! < 2^53) and divided into 1.0 once.
__host__ __device__ constexpr MoeExpCoeffs moe_exp_coeffs() {
  MoeExpCoeffs r{};
  double f = 1.0;
  for (int i = 0; i < 14; ++i) {
    if (i > 1) f *= (double)i;
    r.c[i] = 1.0 / f;
  }
  return r;
}

DEVI double moe_exp64(double z) {
#pragma clang fp contract(off)
  constexpr double kInvLn2 = 1.44269504088896340735992468100189214;   // 1/ln 2
  constexpr double kLn2Hi = 0.693147180559945309417232121458176568;   // ln 2
  constexpr double kLn2Lo = 2.319046813846299558417771e-17;            // ln 2 - kLn2Hi
  constexpr MoeExpCoeffs C = moe_exp_coeffs();
  if (z < -1080.0) return 0.0;
  if (z > 709.0) return __builtin_huge_val();
  double n = __builtin_rint(z * kInvLn2);
  double r = __builtin_fma(-n, kLn2Hi, z);
  r = __builtin_fma(-n, kLn2Lo, r);
  double p = C.c[13];
#pragma unroll
  for (int i = 12; i >= 0; --i) p = __builtin_fma(p, r, C.c[i]);
  return __builtin_ldexp(p, (int)n);
}
