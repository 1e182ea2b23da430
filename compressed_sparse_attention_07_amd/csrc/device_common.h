// Device helpers shared by the gfx950 kernels of libcsa: storage-format
// conversions, RoPE angles, wave-level reductions.  CDNA4 only (wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int v8i32 __attribute__((ext_vector_type(8)));  // 32 fp8 / 64 fp4 codes of an f8f6f4 operand
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;

// ----------------------------------------------------------------- bf16 <-> f32

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even (one v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return static_cast<uint16_t>(pack_bf16x2(f, 0.f) & 0xffffu);
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// --------------------------------------------------------------------- e4m3 (OCP)

// e4m3 code -> float (exact).  0x7f / 0xff decode to NaN.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t s = (c & 0x80u) << 24;
  uint32_t e = (c >> 3) & 0xfu;
  uint32_t m = c & 0x7u;
  if (e == 0xfu && m == 0x7u) return __uint_as_float(0x7fc00000u | s);
  float mag;
  if (e == 0) {
    mag = static_cast<float>(m) * 0.001953125f;  // m * 2^-9
  } else {
    mag = __uint_as_float(((e + 120u) << 23) | (m << 20));  // (1+m/8) * 2^(e-7)
  }
  return __uint_as_float(__float_as_uint(mag) | s);
}

// e4m3 code -> bf16 bits (exact: every e4m3 value is a bf16 value)
__device__ __forceinline__ uint16_t e4m3_to_bf16(uint32_t c) {
  return static_cast<uint16_t>(__float_as_uint(e4m3_to_f32(c)) >> 16);
}

// float -> e4m3 code, nearest-even, saturating to +-448, sign bit follows the input
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  uint32_t u = __float_as_uint(x);
  uint32_t s = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;                   // NaN
  if (a >= 0x43e00000u) return s | 0x7eu;              // |x| >= 448 (incl. inf) -> 448
  int e = static_cast<int>(a >> 23) - 127;             // binade of |x| (normal fp32)
  if (a < 0x00800000u) e = -127;                        // fp32 subnormal: far below range
  if (e < -6) {
    // e4m3 subnormal range: quantum 2^-9, code = rne(|x| / 2^-9)
    float q = __uint_as_float(a) * 512.0f;              // exact scaling by 2^9
    uint32_t r = static_cast<uint32_t>(__builtin_rintf(q));  // rint = nearest-even
    return s | r;                                       // r == 8 is the smallest normal code
  }
  // normal: keep 3 mantissa bits, nearest-even on the 20 dropped bits
  uint32_t mant = a & 0x7fffffu;
  uint32_t keep = mant >> 20;
  uint32_t rest = mant & 0xfffffu;
  uint32_t code = (static_cast<uint32_t>(e + 7) << 3) | keep;
  if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) code += 1;  // may carry into exponent
  if (code > 0x7eu) code = 0x7eu;
  return s | code;
}

// --------------------------------------------------------------------- e2m1 (OCP MX)

__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
  const float mags[8] = {0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f};
  float m = mags[c & 7u];
  return (c & 8u) ? -m : m;
}

// value already divided by the block scale -> 4-bit code, nearest-even, saturating at 6
__device__ __forceinline__ uint32_t f32_to_e2m1(float v) {
  uint32_t s = (__float_as_uint(v) >> 28) & 0x8u;
  float a = fabsf(v);
  uint32_t c;
  // thresholds between neighbours; at an exact midpoint the even code wins
  if (a <= 0.25f) c = 0;
  else if (a < 0.75f) c = 1;
  else if (a <= 1.25f) c = 2;
  else if (a < 1.75f) c = 3;
  else if (a <= 2.5f) c = 4;
  else if (a < 3.5f) c = 5;
  else if (a <= 5.0f) c = 6;
  else c = 7;
  if (a != a) c = 7;  // NaN input: saturate (MX fp4 has no NaN)
  return s | c;
}

// ---------------------------------------------------------------------- RoPE angles

// RoPE angles are formed in fp64 as revolutions (angle / 2pi) and reduced to
// [-1/2, 1/2], then evaluated with the hardware sine / cosine, which take their
// argument in revolutions.  Positions near 2^20 thereby keep full fp32 accuracy
// and the code stays a handful of instructions (no library range reduction).
__device__ __forceinline__ double rope_theta_rev(int j, int R, double log2_base) {
  return exp2(-2.0 * static_cast<double>(j) / static_cast<double>(R) * log2_base) *
         0.15915494309189533576888376337251;  // 1 / (2 pi)
}

__device__ __forceinline__ void rope_cs_rev(double pos, double theta_rev, float* c, float* s) {
  const double r = pos * theta_rev;
  const float f = static_cast<float>(r - rint(r));
  *s = __builtin_amdgcn_sinf(f);
  *c = __builtin_amdgcn_cosf(f);
}

// (cos, sin) of pos * base^(-2j/R)
__device__ __forceinline__ void rope_cs(double pos, int j, int R, double log2_base, float* c, float* s) {
  rope_cs_rev(pos, rope_theta_rev(j, R, log2_base), c, s);
}

// ------------------------------------------------------------------ wave reductions

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

// ---- cross-lane steps without LDS: DPP row shifts inside each 16-lane row, then the
// four row results through readlane.  update_dpp(old, v, row_shr:n, bound_ctrl): a lane
// whose source lies outside its row gets 0 (bound_ctrl) or keeps `old`.
template <int CTRL, bool ZERO>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(static_cast<int>(old), static_cast<int>(v), CTRL, 0xf, 0xf, ZERO));
}
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;

// x combined over the four rows of the wave that share its column (lanes l, l ^ 16,
// l ^ 32, l ^ 48): gfx950's row-swap moves (v_permlane16_swap / v_permlane32_swap) in
// place of two LDS-routed shuffles.  With both operands set to x, the swap leaves x's
// partner row in one output and x in the other in every lane, so each lane combines the
// same pair; both steps are commutative, so every lane ends with the same value.
__device__ __forceinline__ float rows4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float rows4_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// inclusive prefix sum over the 64 lanes
__device__ __forceinline__ uint32_t wave_prefix_sum(uint32_t v) {
  v += dpp_u32<kRowShr1, true>(0u, v);
  v += dpp_u32<kRowShr2, true>(0u, v);
  v += dpp_u32<kRowShr4, true>(0u, v);
  v += dpp_u32<kRowShr8, true>(0u, v);
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
                 r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return v + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// wave-wide reductions; the result is uniform
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  v += dpp_u32<kRowShr1, true>(0u, v);
  v += dpp_u32<kRowShr2, true>(0u, v);
  v += dpp_u32<kRowShr4, true>(0u, v);
  v += dpp_u32<kRowShr8, true>(0u, v);
  return __builtin_amdgcn_readlane(v, 15) + __builtin_amdgcn_readlane(v, 31) + __builtin_amdgcn_readlane(v, 47) +
         __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<kRowShr1, true>(0u, v));
  v = max(v, dpp_u32<kRowShr2, true>(0u, v));
  v = max(v, dpp_u32<kRowShr4, true>(0u, v));
  v = max(v, dpp_u32<kRowShr8, true>(0u, v));
  return max(max(static_cast<uint32_t>(__builtin_amdgcn_readlane(v, 15)), static_cast<uint32_t>(__builtin_amdgcn_readlane(v, 31))),
             max(static_cast<uint32_t>(__builtin_amdgcn_readlane(v, 47)), static_cast<uint32_t>(__builtin_amdgcn_readlane(v, 63))));
}
// float sum and max over the wave by DPP row shifts (no LDS round trips); the result
// is uniform and the order of the additions is fixed
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += __uint_as_float(dpp_u32<kRowShr1, true>(0u, __float_as_uint(v)));
  v += __uint_as_float(dpp_u32<kRowShr2, true>(0u, __float_as_uint(v)));
  v += __uint_as_float(dpp_u32<kRowShr4, true>(0u, __float_as_uint(v)));
  v += __uint_as_float(dpp_u32<kRowShr8, true>(0u, __float_as_uint(v)));
  const float r0 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 15));
  const float r1 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 31));
  const float r2 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 47));
  const float r3 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 63));
  return (r0 + r1) + (r2 + r3);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v);
// max of non-NaN floats through their order-preserving integer images
__device__ __forceinline__ float wave_max_dpp(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t k = wave_max_u32((u & 0x80000000u) ? ~u : (u | 0x80000000u));
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_u32<kRowShr1, false>(0xffffffffu, v));
  v = min(v, dpp_u32<kRowShr2, false>(0xffffffffu, v));
  v = min(v, dpp_u32<kRowShr4, false>(0xffffffffu, v));
  v = min(v, dpp_u32<kRowShr8, false>(0xffffffffu, v));
  return min(min(static_cast<uint32_t>(__builtin_amdgcn_readlane(v, 15)), static_cast<uint32_t>(__builtin_amdgcn_readlane(v, 31))),
             min(static_cast<uint32_t>(__builtin_amdgcn_readlane(v, 47)), static_cast<uint32_t>(__builtin_amdgcn_readlane(v, 63))));
}

// ---- loads of data read once (a stream no other workgroup of the launch reads again):
// the nontemporal hint keeps them from displacing data that is reused

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(x.x, x.y, x.z, x.w);
}

// ---- direct global -> LDS loads
//
// One 16-byte-per-lane load to LDS (global_load_lds_dwordx4): lane i's 16 bytes land at
// M0 + 16 i.  Used for 1 KiB rows / row groups.  M0 is saved and restored around the instruction (the address
// is taken at issue), so the compiler's own uses of M0 are unaffected.
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds_byte) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(g), "s"(lds_byte)
               : "memory");
}

// The same with the nontemporal hint, for rows that no other workgroup of the launch
// reads again (a key stream scored once).
__device__ __forceinline__ void lds_dma16_nt(const void* g, uint32_t lds_byte) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(g), "s"(lds_byte)
               : "memory");
}

// The same for one dword per lane: the wave's 64 dwords land contiguously at lds_byte.
__device__ __forceinline__ void lds_dma4(const void* g, uint32_t lds_byte) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(g), "s"(lds_byte)
               : "memory");
}

// Workgroups go to the 8 XCDs round-robin (block b runs on XCD b % 8), and each XCD
// has its own L2.  This renumbering hands every XCD one contiguous range of logical
// blocks, so blocks that read the same data (splits of one query token, neighbouring
// tokens' overlapping selections) meet in one L2.  A tail of grid % 8 blocks keeps its
// own numbers.
__device__ __forceinline__ uint32_t xcd_block(uint32_t b, uint32_t grid) {
  constexpr uint32_t kXcd = 8;
  const uint32_t full = grid - grid % kXcd;
  return b < full ? (b % kXcd) * (full / kXcd) + b / kXcd : b;
}

// a wave-uniform 64-bit value, moved to scalar registers
__device__ __forceinline__ int64_t uni64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(x) >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <typename T>
__device__ __forceinline__ T ceil_div(T a, T b) {
  return (a + b - 1) / b;
}

// Order-preserving map of a finite float to uint32 (larger float -> larger key;
// -0 and +0 map to the same key).  Non-finite inputs (inf, NaN) map to 0, which no
// finite value reaches.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Paged compressed caches ([V4-CN] §3.6.1): entry e of the sequence in batch row b lives
// at pool row  table[slot[b] * max_pages + (e >> shift)] << shift | (e & (2^shift - 1)).
// table == NULL: unpaged, row b * rows_per_seq + e.
struct PageMap {
  const int32_t* table;  // [slots, max_pages] page of each block of 2^shift entries
  const int32_t* slot;   // [B] state slot of each batch row
  int max_pages, shift;
};

__device__ __forceinline__ int64_t paged_row(const PageMap& m, int64_t b, int64_t e) {
  const int64_t page = m.table[static_cast<int64_t>(m.slot[b]) * m.max_pages + (e >> m.shift)];
  return (page << m.shift) | (e & ((int64_t{1} << m.shift) - 1));
}

}  // namespace csa
