// device.h -- device helpers shared by the kernel sources: vector types, segment bounds,
// buffer resources, the bf16 matrix-core product and lane exchanges.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace fmha {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;

struct Seg {
  int64_t q_row0;   // first tensor row of the segment (0 in batch mode)
  int64_t k_row0;
  int64_t lq, lk;   // segment lengths
  int64_t ws_row0;  // first workspace row of D and LSE2 (b*Sq in batch mode)
  int64_t acc_row0; // first accumulator row: ws_row0 + b*acc_pad
  int64_t kws_row0; // first key row of the dK/dV partials (b*Sk in batch mode)
};

// Segment bounds; b is uniform across the work group and readfirstlane keeps the loaded
// offsets in scalar registers, so everything derived from them stays wave-uniform.
__device__ __forceinline__ Seg seg_of(const KParams& p, int b) {
  Seg s;
  if (p.seqstart_q != nullptr) {
    const int q0 = __builtin_amdgcn_readfirstlane(p.seqstart_q[b]);
    const int q1 = __builtin_amdgcn_readfirstlane(p.seqstart_q[b + 1]);
    const int k0 = __builtin_amdgcn_readfirstlane(p.seqstart_k[b]);
    const int k1 = __builtin_amdgcn_readfirstlane(p.seqstart_k[b + 1]);
    s.q_row0 = p.slot_q ? __builtin_amdgcn_readfirstlane(p.slot_q[b]) : q0;
    s.lq = (int64_t)q1 - q0;
    s.k_row0 = p.slot_k ? __builtin_amdgcn_readfirstlane(p.slot_k[b]) : k0;
    s.lk = (int64_t)k1 - k0;
    s.ws_row0 = s.q_row0;
    s.kws_row0 = s.k_row0;
  } else {
    s.q_row0 = 0;
    s.k_row0 = 0;
    s.lq = p.Sq;
    s.lk = p.Sk;
    s.ws_row0 = (int64_t)b * p.Sq;
    s.kws_row0 = (int64_t)b * p.Sk;
  }
  s.acc_row0 = s.ws_row0 + (int64_t)b * p.acc_pad;
  return s;
}

// Element offset of (segment b, tensor row `row`, head h, column 0).
__device__ __forceinline__ int64_t elem_off(const int64_t s[3], bool group, int b, int64_t row,
                                            int h) {
  return (group ? 0 : (int64_t)b * s[0]) + row * s[1] + (int64_t)h * s[2];
}

__device__ __forceinline__ bf16x8 tr_read(const uint16_t* p0, const uint16_t* p1) {
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p0));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p1));
  const s16x8 c = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

// Raw buffer resource over [base, base + bytes): loads past the end return 0 and stores or
// atomics past the end are dropped by the hardware range check.  Callers pass every offset in
// the per-lane offset operand and 0 as the scalar offset.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Cache-policy operand of the buffer loads and stores of the deterministic dQ partials: the
// non-temporal bit, so that the partials (written once, read back once) stream through the
// caches instead of displacing the Q, K, V and dO tiles that other work groups re-read.  The
// dK/dV partials of split key tiles use the same policy through the non-temporal builtins.
// Measured on one MI355X: the causal 2 x 32 x 4096 deterministic step 1.05 -> 0.99 ms, the
// 8192-token ragged GQA one 0.556 -> 0.506 ms.
constexpr int kPartialPolicy = 2;

// The lane index, read again where it is used: a volatile asm statement is not hoisted out of
// a loop, so per-lane values derived from it are computed where they are needed instead of
// being kept live (and spilled) across the main kernels' step loops.
__device__ __forceinline__ int lane_here() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint16_t to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// Key (inside the wave's 32) held by lane l32: bit 4 of the lane is bit 0 of the key and lane
// bits 0..3 are key bits 1..4.  With it the dS exchange below ends with lane bits 2, 3 naming
// an aligned group of 8 keys and the exchanged register bits naming the key inside the group.
__device__ __forceinline__ int kmap(int l) {
  return ((l >> 4) & 1) | ((l & 15) << 1);
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(unsigned, bf16x2{(__bf16)lo, (__bf16)hi});
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3",
// SC 2011) of counter c under key (k0, k1), in place.  The dropout keep mask of element
// (b, h, i, j) is byte (j % 4) of output word (i % 4) for counter (j/4, i/4, b*Hq + h, offset).
__device__ __forceinline__ void philox4x32_10(unsigned (&c)[4], unsigned k0, unsigned k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    const unsigned n0 = (unsigned)(p1 >> 32) ^ c[1] ^ k0;
    const unsigned n2 = (unsigned)(p0 >> 32) ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = (unsigned)p1;
    c[2] = n2;
    c[3] = (unsigned)p0;
  }
}

// 4x4 byte transpose: t[k] holds byte k of w[0], w[1], w[2], w[3] in its bytes 0..3.
__device__ __forceinline__ void byte_transpose4(const unsigned (&w)[4], unsigned (&t)[4]) {
  const unsigned a0 = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);  // w0.0 w1.0 w0.1 w1.1
  const unsigned a1 = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);  // w0.2 w1.2 w0.3 w1.3
  const unsigned b0 = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u);  // w2.0 w3.0 w2.1 w3.1
  const unsigned b1 = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);  // w2.2 w3.2 w2.3 w3.3
  t[0] = __builtin_amdgcn_perm(b0, a0, 0x05040100u);
  t[1] = __builtin_amdgcn_perm(b0, a0, 0x07060302u);
  t[2] = __builtin_amdgcn_perm(b1, a1, 0x05040100u);
  t[3] = __builtin_amdgcn_perm(b1, a1, 0x07060302u);
}

__device__ __forceinline__ unsigned sel4(const unsigned (&v)[4], unsigned i) {
  return (i & 2u) ? ((i & 1u) ? v[3] : v[2]) : ((i & 1u) ? v[1] : v[0]);
}

// Value of lane (l ^ 1) and of lane (l ^ 2) (DPP quad permutations).
__device__ __forceinline__ unsigned xor1(unsigned v) {
  return (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);
}
__device__ __forceinline__ unsigned xor2(unsigned v) {
  return (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);
}
__device__ __forceinline__ unsigned xor3(unsigned v) {
  return (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x1B, 0xF, 0xF, true);
}
// Value of lane (l ^ 16): v_permlane16_swap of v with itself leaves lane l ^ 16's value in
// the second result for lanes with bit 4 clear and in the first for the others.
__device__ __forceinline__ unsigned xor16(unsigned v, int lane) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return (lane & 16) ? r[0] : r[1];
}

}  // namespace
}  // namespace fmha
