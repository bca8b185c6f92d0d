// Device-side helpers shared by the GEMV kernels: vector types, bit casts, the
// x pair order of the nibble decode, DPP / lane-swap team sums, the lane
// transpose of the MFMA B layout, LDS waits, the buffer cache-policy bits and
// the subnormal-code group dot product of the persistent kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_g __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3_g __attribute__((ext_vector_type(3)));
typedef uint32_t u32x4_g __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8_s __attribute__((ext_vector_type(8)));

// Pointers read from a descriptor table are generic; casting them to the global
// address space makes the compiler emit global_* (not flat_*) memory
// instructions, which count only in vmcnt (flat ones also count in lgkmcnt, so
// every LDS wait would also wait for the weight stream).
#define Q4_GLOBAL __attribute__((address_space(1)))

// Buffer-instruction cache policy bits and the raw-buffer resource flags.
constexpr int kCoherent = 1 | 16;        // sc0 | sc1: device-coherent access
constexpr int kNonTemporal = 2;          // nt: streamed once
constexpr int kRsrcFlags = 0x00020000;   // raw buffer, 32-bit data format
constexpr int kWaitVm0 = 0x0F70;         // s_waitcnt vmcnt(0) (expcnt, lgkmcnt untouched)

template <typename T, typename F>
__device__ __forceinline__ T bits(F v) {
  return __builtin_bit_cast(T, v);
}

__device__ __forceinline__ float half_to_float(uint16_t h) { return (float)bits<_Float16>(h); }

__device__ __forceinline__ uint16_t float_to_half_rne(float v) {
  return bits<uint16_t>((_Float16)v);
}

// A block of 8 consecutive x values (one word's worth) reordered into the pairs
// (x0,x4) (x1,x5) (x2,x6) (x3,x7) in which a word's nibble pairs are decoded.
__device__ __forceinline__ uint4 pair_order(uint4 v) {
  uint4 o;
  o.x = (v.x & 0xFFFFu) | (v.z << 16);
  o.y = (v.x >> 16) | (v.z & 0xFFFF0000u);
  o.z = (v.y & 0xFFFFu) | (v.w << 16);
  o.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
  return o;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return bits<float>(__builtin_amdgcn_update_dpp(0, bits<int>(v), CTRL, 0xF, 0xF, true));
}

// Sum over aligned teams of 2^lg lanes (lg in [2, 6], uniform over the wave);
// every lane of a team gets the total.  No LDS, no barrier.
__device__ __forceinline__ float team_sum_lg(float v, int lg) {
  v += dpp<0xB1>(v);                   // quad_perm [1,0,3,2]: lane ^ 1
  v += dpp<0x4E>(v);                   // quad_perm [2,3,0,1]: lane ^ 2
  if (lg >= 3) v += dpp<0x141>(v);     // row_half_mirror: the other quad
  if (lg >= 4) v += dpp<0x140>(v);     // row_mirror: the other half-row
  if (lg >= 5) {                       // rows 0<->1 and 2<->3
    const auto r = __builtin_amdgcn_permlane16_swap(bits<uint32_t>(v), bits<uint32_t>(v),
                                                    false, false);
    v = bits<float>((uint32_t)r[0]) + bits<float>((uint32_t)r[1]);
  }
  if (lg >= 6) {                       // lanes 0-31 <-> 32-63
    const auto r = __builtin_amdgcn_permlane32_swap(bits<uint32_t>(v), bits<uint32_t>(v),
                                                    false, false);
    v = bits<float>((uint32_t)r[0]) + bits<float>((uint32_t)r[1]);
  }
  return v;
}

// The same for a team size known at compile time.
template <int LPR>
__device__ __forceinline__ float team_sum(float v) {
  static_assert(LPR == 4 || LPR == 8 || LPR == 16 || LPR == 32 || LPR == 64, "team size");
  return team_sum_lg(v, LPR == 4 ? 2 : LPR == 8 ? 3 : LPR == 16 ? 4 : LPR == 32 ? 5 : 6);
}

// A 4 x 4 block spread over lanes r, r+16, r+32, r+48: rows {0,1} <-> {2,3}, then
// rows 0 <-> 1 and 2 <-> 3; afterwards lane row R register t holds what lane row t
// register R held.
__device__ __forceinline__ void transpose4(uint32_t (&v)[4]) {
  auto a = __builtin_amdgcn_permlane32_swap(v[0], v[2], false, false);
  auto b = __builtin_amdgcn_permlane32_swap(v[1], v[3], false, false);
  v[0] = a[0]; v[2] = a[1]; v[1] = b[0]; v[3] = b[1];
  auto c = __builtin_amdgcn_permlane16_swap(v[0], v[1], false, false);
  auto d = __builtin_amdgcn_permlane16_swap(v[2], v[3], false, false);
  v[0] = c[0]; v[1] = c[1]; v[2] = d[0]; v[3] = d[1];
}

// s_waitcnt lgkmcnt(0) only: this wave's LDS operations are complete; its
// outstanding vector-memory loads are not waited for.
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

__device__ __forceinline__ int lds_load(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ void lds_store(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// The nibble-pair masks.  AND-ing a word with 0x000F000F leaves nibbles 0 and 4
// as the mantissas of two fp16 subnormals, the exact values (q0, q4) * 2^-24;
// with 0x00F000F0, nibbles 1 and 5 sit one mantissa position higher, (q1, q5) *
// 2^-20; the same on word >> 8 gives elements 2, 6 and 3, 7.  Each pair is ONE
// v_and_b32, with no exponent to insert and no offset to remove: the zero point
// is taken off once per group (see nibble_group_dot).  The masks live in VGPRs.
struct Nibbles {
  uint32_t m_lo, m_hi;   // 0x000F000F, 0x00F000F0
};

__device__ __forceinline__ Nibbles make_nibbles() {
  Nibbles n{0x000F000Fu, 0x00F000F0u};
  asm volatile("" : "+v"(n.m_lo), "+v"(n.m_hi));
  return n;
}

// One 32-weight group: 2^-20 * sum_k q_k x_k in fp32, from the codes as fp16
// subnormals (products exact in fp32) and two chains of v_dot2, even and odd
// positions, joined as 16 * even + odd (exact scaling).  x holds the group's
// four pair-ordered blocks.  The wanted 2^-20 * sum_k (q_k - 7) x_k is this minus
// the same function of a word whose codes are all 7 (0x77777777) with the same x,
// which the sync waves compute once per group when they stage x: both are the
// same instructions on the same operands, so a group of codes 7 gives exactly
// zero, and integer codes and x give the exact integer.  The factor 2^20 is
// applied to the row's sum.
__device__ __forceinline__ float nibble_group_dot(uint4 w, const uint4 (&x)[4],
                                                  const Nibbles& nb) {
  const uint32_t wj[4] = {w.x, w.y, w.z, w.w};
  // the first product of each chain in the three-operand form: the compiler
  // would otherwise copy the start value into the accumulator of v_dot2c
  float a, b;
  {
    const uint32_t v = wj[0];
    asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(a) : "v"(v & nb.m_lo), "v"(x[0].x));
    asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(b) : "v"(v & nb.m_hi), "v"(x[0].y));
    const uint32_t v8 = v >> 8;
    a = __builtin_amdgcn_fdot2(bits<h2_t>(v8 & nb.m_lo), bits<h2_t>(x[0].z), a, false);
    b = __builtin_amdgcn_fdot2(bits<h2_t>(v8 & nb.m_hi), bits<h2_t>(x[0].w), b, false);
  }
#pragma unroll
  for (int j = 1; j < 4; ++j) {
    const uint32_t v = wj[j], v8 = v >> 8;
    a = __builtin_amdgcn_fdot2(bits<h2_t>(v & nb.m_lo), bits<h2_t>(x[j].x), a, false);
    b = __builtin_amdgcn_fdot2(bits<h2_t>(v & nb.m_hi), bits<h2_t>(x[j].y), b, false);
    a = __builtin_amdgcn_fdot2(bits<h2_t>(v8 & nb.m_lo), bits<h2_t>(x[j].z), a, false);
    b = __builtin_amdgcn_fdot2(bits<h2_t>(v8 & nb.m_hi), bits<h2_t>(x[j].w), b, false);
  }
  return __builtin_fmaf(a, 16.f, b);
}

// 2^20: the factor between nibble_group_dot's units and the products' (exact in fp32).
constexpr float kDotUnit = 1048576.f;

// q3f16_1: the codes become fp16 pairs without extracting them one by one.  A
// 32-bit window of a group's 96-bit value, taken at bit 3i - 4 (one shift or
// funnel shift), holds code i at bits 4-6, code i+1 at 7-9, code i+4 at 16-18
// and code i+5 at 19-21.  Masking two of those fields and OR-ing in an exponent
// chosen per field so that the field's lowest bit has place value 1 gives fp16
// values 2^E + q exactly (E = 6, 3, 10, 7 for the four fields), one AND-OR per
// pair; v_dot2_f32_f16 multiplies a pair by the matching x pair.  Per group the
// sum of (2^E + 3) * x over its codes is staged beside x and subtracted once,
// which leaves sum (q - 3) * x.  Windows at i = 0, 2, 8, 10, 16, 18, 24, 26
// cover the 32 codes as the pairs (i, i+4), (i+1, i+5).
constexpr uint32_t kQ3MaskA = 0x00070070u, kQ3MaskB = 0x00380380u;
constexpr uint32_t kQ3ExpA = 0x64005400u, kQ3ExpB = 0x58004800u;


// Sum over one group of (2^E + q) * x.  xq: x of the group as four chunks of
// four pairs, chunk c at xq[c * cstride] holding the pairs (x[8c+p], x[8c+p+4]).
// ma, mb: kQ3MaskA and kQ3MaskB held in registers (an instruction with three
// operands takes no literal constant, and two literals would split each AND-OR
// into two instructions).
__device__ __forceinline__ float q3_group_dot(uint32_t w0, uint32_t w1, uint32_t w2,
                                              const uint4* xq, int cstride, uint32_t ma,
                                              uint32_t mb) {
  const uint32_t v[8] = {w0 << 4,
                         __builtin_amdgcn_alignbit(w1, w0, 2),
                         __builtin_amdgcn_alignbit(w1, w0, 20),
                         __builtin_amdgcn_alignbit(w1, w0, 26),
                         __builtin_amdgcn_alignbit(w2, w1, 12),
                         __builtin_amdgcn_alignbit(w2, w1, 18),
                         w2 >> 4,
                         w2 >> 10};
  float a = 0.f, b = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint4 xv = xq[c * cstride];
    a = __builtin_amdgcn_fdot2(bits<h2_t>((v[2 * c] & ma) | kQ3ExpA), bits<h2_t>(xv.x), a, false);
    b = __builtin_amdgcn_fdot2(bits<h2_t>((v[2 * c] & mb) | kQ3ExpB), bits<h2_t>(xv.y), b, false);
    a = __builtin_amdgcn_fdot2(bits<h2_t>((v[2 * c + 1] & ma) | kQ3ExpA), bits<h2_t>(xv.z), a,
                               false);
    b = __builtin_amdgcn_fdot2(bits<h2_t>((v[2 * c + 1] & mb) | kQ3ExpB), bits<h2_t>(xv.w), b,
                               false);
  }
  return a + b;
}

// The same for x held in registers (the four pair-ordered blocks of the group).
__device__ __forceinline__ float q3_group_dot(uint32_t w0, uint32_t w1, uint32_t w2,
                                              const uint4 (&x)[4], uint32_t ma, uint32_t mb) {
  const uint32_t v[8] = {w0 << 4,
                         __builtin_amdgcn_alignbit(w1, w0, 2),
                         __builtin_amdgcn_alignbit(w1, w0, 20),
                         __builtin_amdgcn_alignbit(w1, w0, 26),
                         __builtin_amdgcn_alignbit(w2, w1, 12),
                         __builtin_amdgcn_alignbit(w2, w1, 18),
                         w2 >> 4,
                         w2 >> 10};
  float a = 0.f, b = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint4 xv = x[c];
    a = __builtin_amdgcn_fdot2(bits<h2_t>((v[2 * c] & ma) | kQ3ExpA), bits<h2_t>(xv.x), a, false);
    b = __builtin_amdgcn_fdot2(bits<h2_t>((v[2 * c] & mb) | kQ3ExpB), bits<h2_t>(xv.y), b, false);
    a = __builtin_amdgcn_fdot2(bits<h2_t>((v[2 * c + 1] & ma) | kQ3ExpA), bits<h2_t>(xv.z), a,
                               false);
    b = __builtin_amdgcn_fdot2(bits<h2_t>((v[2 * c + 1] & mb) | kQ3ExpB), bits<h2_t>(xv.w), b,
                               false);
  }
  return a + b;
}

// A q3f16_1 group whose 32 codes are all 3 (the zero point), as its three
// little-endian words: q3_group_dot of it with a group's x is the offset term
// that leaves sum (q - 3) x, formed with the same instructions as the group's
// own dot product, so codes 3 give exactly zero.
constexpr uint32_t kQ3Zero0 = 0xDB6DB6DBu, kQ3Zero1 = 0xB6DB6DB6u, kQ3Zero2 = 0x6DB6DB6Du;

}  // namespace q4
