// Device building blocks for gfx950: trellis decode into MFMA B operands,
// the MCG16 codebook on packed 16-bit lanes, a 128-point FWHT on 16-lane
// groups, and the v_mfma_f32_16x16x32_f16 wrapper.
//
// Format (this library's definition; the pages name trellis widths and the
// MCG codebook but define neither — exllamav3 PR #284 "MoE: Add fused
// additive EXL3 kernels", API contract; TensorFold PR #837, What this
// changes):
//   CB(s)  = (-1)^h[15] * 2^(h[11:10] - 3) * (1 + h[9:0]/1024),
//            h = s * 0x9E37 mod 2^16; as fp16 bits: (h & 0x8FFF) | 0x3000
//   tile   16 (k) x 16 (n) weights, 256*K-bit tail-biting stream; the state of
//          weight i is the 16 stream bits ending at bit i*K + K - 1; weight i
//          sits at (k = i mod 16, n = i / 16)
//   tensor uint16 [out/16][in/16][16K], tile (kt, nt) at (nt*in/16 + kt)*16K
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace exl3 {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// Global-address-space views (keeps loads on the global_load path).
typedef const uint32_t __attribute__((address_space(1))) *gu32p;
typedef const u32x4 __attribute__((address_space(1))) *gu32x4p;

constexpr float kRsqrt128 = 0.08838834764831845f;  // 1/sqrt(128), fp32

// GPU-internal k order of rotated activations: inside every aligned group of
// 16 entries, stored slot p holds entry kSigma[p] =
// {0,4,1,5,2,6,3,7, 8,12,9,13,10,14,11,15}. It matches the order in which one
// lane's decoded B values reach the MFMA (see decode_half).
// Entry k (0..15) of a 16-group -> stored slot.
__device__ __forceinline__ int sigma_inv(int k) {
  // inverse of kSigma: k -> 2*(k&3) + ((k>>2)&1) + (k&8)
  return ((k & 3) << 1) | ((k >> 2) & 1) | (k & 8);
}

// ---------------------------------------------------------------- codebook
// Two MCG16 states in the 16-bit halves of s2 -> two fp16 codebook values.
// Bit 15 of h is the fp16 sign, bits 10..11 the low exponent bits under a
// fixed 0b011 (exponent 12..15), bits 0..9 the mantissa: one
// v_pk_mul_lo_u16 and one v_and_or_b32 (mask in a VGPR, OR constant in an
// SGPR) per two weights.
__device__ __forceinline__ uint32_t codebook2(uint32_t s2, uint32_t mask) {
  u16x2 s = __builtin_bit_cast(u16x2, s2);
  u16x2 h = s * (u16x2){(unsigned short)0x9E37, (unsigned short)0x9E37};
  return (__builtin_bit_cast(uint32_t, h) & mask) | 0x30003000u;
}

// A VGPR holding 0x8FFF8FFF that the compiler cannot fold back into a literal
// (gfx9 VOP3 encodings take no literal operand).
__device__ __forceinline__ uint32_t codebook_mask() {
  uint32_t m;
  asm volatile("v_mov_b32 %0, 0x8fff8fff" : "=v"(m));
  return m;
}

// ------------------------------------------------------------ tile geometry
template <int K>
struct Geom {
  static constexpr int kTileDw = 8 * K;  // dwords per tile
};

// Geometry of half a tile column (8 consecutive states): the window is
// 7K + 16 bits long.
template <int K>
struct HalfGeom {
  static constexpr int kLoadDw = (7 * K + 16 + 31 + 31) / 32;  // at any bit offset
  static constexpr int kNormDw = (7 * K + 16 + 31) / 32;       // shifted to bit 0
};

// 32 bits of a normalised window N starting at bit OFF (bits < 0 read 0).
template <int OFF, int NN>
__device__ __forceinline__ uint32_t window32(const uint32_t (&N)[NN]) {
  if constexpr (OFF < 0) {
    return N[0] << (-OFF);
  } else {
    constexpr int w = OFF >> 5, s = OFF & 31;
    const uint32_t lo = N[w];
    if constexpr (s == 0) {
      return lo;
    } else {
      const uint32_t hi = (w + 1 < NN) ? N[(w + 1 < NN) ? w + 1 : w] : 0u;
      return __builtin_amdgcn_alignbit(hi, lo, s);
    }
  }
}

// Dword D of a normalised window, 0 past its end.
template <int D, int NN>
__device__ __forceinline__ uint32_t norm_dw(const uint32_t (&N)[NN]) {
  if constexpr (D < NN) return N[D];
  else return 0u;
}

// Raw dwords of a window (ND of them, the window starting at bit `shift` of
// raw[0]) shifted down to bit 0 (NN dwords).
template <int ND, int NN>
__device__ __forceinline__ void normalize(const uint32_t (&raw)[ND], uint32_t shift,
                                          uint32_t (&N)[NN]) {
#pragma unroll
  for (int j = 0; j < NN; ++j) {
    const uint32_t hi = (j + 1 < ND) ? raw[(j + 1 < ND) ? j + 1 : j] : 0u;
    N[j] = __builtin_amdgcn_alignbit(hi, raw[j], shift);
  }
}

// States (j, j + 4) of a normalised window (state i starting at bit iK) in
// the low and high 16-bit halves of one dword (bits above a state's 16 are
// don't-care for the 16-bit hash). State j starts at bit o1 = jK, state
// j + 4 at o2 = o1 + 4K. Chosen per (K, j) at compile time:
//   4K == 16          one funnel shift (K = 4)
//   both byte-aligned one or two byte permutes of the window dwords (K = 8;
//                     K = 6 and K = 2 for j = 0 mod 4)
//   4K == 8           one funnel shift and a byte permute (K = 2)
//   otherwise         two funnel shifts and a byte permute
// v_perm_b32 byte selector s picks byte s of {hi, lo} (0..3 from lo).
template <int K, int j, int NN>
__device__ __forceinline__ uint32_t column_pair(const uint32_t (&N)[NN]) {
  constexpr int o1 = j * K, o2 = (j + 4) * K;
  if constexpr (o2 - o1 == 16) {
    return window32<o1>(N);
  } else if constexpr (o1 % 8 == 0 && o2 % 8 == 0) {
    constexpr int w = o1 / 32;
    constexpr uint32_t b1 = o1 / 8 - 4 * w, b2 = o2 / 8 - 4 * w;
    if constexpr (b2 + 1 <= 7) {
      constexpr uint32_t sel = b1 | ((b1 + 1) << 8) | (b2 << 16) | ((b2 + 1) << 24);
      return __builtin_amdgcn_perm(norm_dw<w + 1>(N), N[w], sel);
    } else {
      // b2 = 7: byte b2 + 1 is byte 0 of dword w + 2
      constexpr uint32_t sel1 = b1 | ((b1 + 1) << 8) | (b2 << 16) | (b2 << 24);
      const uint32_t t = __builtin_amdgcn_perm(norm_dw<w + 1>(N), N[w], sel1);
      return __builtin_amdgcn_perm(norm_dw<w + 2>(N), t, 0x04020100u);
    }
  } else if constexpr (o2 - o1 == 8) {
    const uint32_t x = window32<o1>(N);
    return __builtin_amdgcn_perm(x, x, 0x02010100u);
  } else {
    const uint32_t lo = window32<o1>(N);
    const uint32_t hi = window32<o2 - 16>(N);
    return __builtin_amdgcn_perm(hi, lo, 0x07060100u);
  }
}

// Register r (0..3) of a decoded half column (window normalised to its first
// state): states (r, r + 4) of the half, fp16 k-slots {0,4,1,5,2,6,3,7}.
template <int K, int r, int NN>
__device__ __forceinline__ uint32_t half_reg(const uint32_t (&N)[NN], uint32_t mask) {
  return codebook2(column_pair<K, r>(N), mask);
}

// K = 4 and K = 8: the first state of every half column starts at the same
// bit of the half column's first loaded dword (20 for K = 4, 24 for K = 8:
// 16nK + 8hK + K - 16 is 20 resp. 24 mod 32 for every column n and half h),
// so the state pairs are cut straight from the loaded dwords with
// compile-time shifts and byte selectors, with no per-lane normalisation.
template <int K>
constexpr bool kRawPairs = (K == 4 || K == 8);

// Register r (0..3) of a decoded half column from its loaded dwords (K = 4
// or 8): states (r, r + 4), as half_reg.
template <int K, int r, int ND>
__device__ __forceinline__ uint32_t half_reg_raw(const uint32_t (&raw)[ND], uint32_t mask) {
  static_assert(kRawPairs<K>, "constant window start only for K = 4, 8");
  uint32_t pair;
  if constexpr (K == 4) {
    // states r, r + 4 = the 32 bits from bit 20 + 4r
    constexpr int o = 20 + 4 * r, w = o >> 5, sh = o & 31;
    if constexpr (sh == 0) pair = raw[w];
    else pair = __builtin_amdgcn_alignbit(raw[w + 1], raw[w], sh);
  } else {
    // state r = bytes 3 + r, 4 + r; state r + 4 = bytes 7 + r, 8 + r
    if constexpr (r == 0) {
      const uint32_t t = __builtin_amdgcn_perm(raw[1], raw[0], 0x07070403u);  // b3 b4 b7 b7
      pair = __builtin_amdgcn_perm(raw[2], t, 0x04020100u);                      // b8 in byte 3
    } else {
      constexpr uint32_t a = r - 1;  // bytes 4 + r.. of raw[1] are bytes a.. of it
      constexpr uint32_t sel = a | ((a + 1) << 8) | ((a + 4) << 16) | ((a + 5) << 24);
      pair = __builtin_amdgcn_perm(raw[2], raw[1], sel);
    }
  }
  return codebook2(pair, mask);
}

// The half column a lane decodes in one 32-input MFMA k-step (two tiles along
// k): lane (g, n) takes states 8h .. 8h + 7 (h = g & 1) of column n of tile
// t = g >> 1, i.e. the 8 k-entries it feeds the MFMA. Their window starts at
// bit 16nK + 8hK + K - 16 of tile t's tail-biting stream. off[j] is the byte
// offset of the window's dword j from the step's first tile (tile t's own
// base included, wrapped inside the tile); shift is the window's bit offset
// inside dword 0. Every kernel that decodes trellis (both GEMM tile shapes and
// the diagnostic decode export) takes its addresses from here.
template <int K>
struct HalfWindow {
  static constexpr int ND = HalfGeom<K>::kLoadDw;
  uint32_t off[ND];
  uint32_t shift;
  __device__ __forceinline__ explicit HalfWindow(int lane) {
    constexpr int TD = Geom<K>::kTileDw;
    const int g = lane >> 4, n = lane & 15;
    const int b = 16 * n * K + 8 * (g & 1) * K + K - 16;
    const int d0 = b >> 5;  // floor
    shift = (uint32_t)(b & 31);
#pragma unroll
    for (int j = 0; j < ND; ++j) {
      int d = d0 + j;
      d += (d < 0) ? TD : 0;
      d -= (d >= TD) ? TD : 0;
      off[j] = (uint32_t)((g >> 1) * TD + d) * 4u;
    }
  }
};

// Register r (0..3) of a decoded half column from the raw window dwords:
// states (r, r + 4), fp16 k-slots {2r, 2r + 1} of the lane's MFMA operand.
// K = 4 and 8 cut the pairs straight from the raw dwords; other widths shift
// the window to bit 0 first (N, computed when r == 0 and reused for r > 0).
template <int K, int r>
__device__ __forceinline__ uint32_t half_column_reg(const uint32_t (&raw)[HalfGeom<K>::kLoadDw],
                                                    uint32_t shift,
                                                    uint32_t (&N)[HalfGeom<K>::kNormDw],
                                                    uint32_t mask) {
  if constexpr (kRawPairs<K>) {
    (void)shift;
    (void)N;
    return half_reg_raw<K, r>(raw, mask);
  } else {
    if constexpr (r == 0) normalize(raw, shift, N);
    return half_reg<K, r>(N, mask);
  }
}

// The whole decoded half column: the 8 fp16 B-operand values of the lane.
template <int K>
__device__ __forceinline__ u32x4 decode_half(const uint32_t (&raw)[HalfGeom<K>::kLoadDw],
                                             uint32_t shift, uint32_t mask) {
  uint32_t N[HalfGeom<K>::kNormDw];
  const uint32_t r0 = half_column_reg<K, 0>(raw, shift, N, mask);
  const uint32_t r1 = half_column_reg<K, 1>(raw, shift, N, mask);
  const uint32_t r2 = half_column_reg<K, 2>(raw, shift, N, mask);
  const uint32_t r3 = half_column_reg<K, 3>(raw, shift, N, mask);
  return (u32x4){r0, r1, r2, r3};
}

// Wave index as a scalar: lets the compiler keep every per-wave value (and
// the buffer resources built from them) in SGPRs.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// Loads of per-workgroup / per-wave table entries (plan tiles, stage
// tables) as scalar loads: the address is made uniform and read through the
// constant address space, so the value lands in SGPRs through the scalar
// cache. Only for data written before the kernel started (the scalar cache is
// not coherent with stores of the same launch).
template <typename T>
__device__ __forceinline__ T sload(const T *a) {
  const uint64_t b = (uint64_t)(uintptr_t)a;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  typedef const T __attribute__((address_space(4))) *cptr;
  return *(cptr)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ int uload_i32(const int32_t *a) { return sload(a); }
__device__ __forceinline__ float uload_f32(const float *a) { return sload(a); }
__device__ __forceinline__ const uint32_t *uload_ptr(const int64_t *a) {
  return (const uint32_t *)(uintptr_t)sload(a);
}

// -------------------------------------------------------------------- MFMA
// D[16x16] += A[16x32] * B[32x16], fp16 inputs, fp32 accumulate. Lane l
// supplies A row (l & 15) and B column (l & 15), 8 k-entries each for the
// k-group l >> 4; it receives D rows 4*(l>>4) + r (r = 0..3), column l & 15.
__device__ __forceinline__ f32x4 mfma16x16x32(const f16x8 &a, const f16x8 &b,
                                              const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// --------------------------------------------------------------------- FWHT
// Unnormalised 128-point Walsh-Hadamard transform (Sylvester order) on a
// group of 16 consecutive lanes; lane i of the group holds entries
// i + 16*j in v[j]. Butterflies (lo, hi) -> (lo + hi, lo - hi), distances
// 1, 2, 4, 8 across lanes then 16, 32, 64 in registers. The fixed order makes
// the fp32 result a pure function of the inputs.
__device__ __forceinline__ void fwht128_group16(float (&v)[8]) {
  const int i = threadIdx.x & 15;
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) {
    const bool upper = (i & d) != 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float o = __shfl_xor(v[j], d, 64);
      v[j] = upper ? (o - v[j]) : (v[j] + o);
    }
  }
#pragma unroll
  for (int d = 1; d < 8; d <<= 1) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if ((j & d) == 0) {
        const float lo = v[j], hi = v[j + d];
        v[j] = lo + hi;
        v[j + d] = lo - hi;
      }
    }
  }
}

constexpr double kRsqrt128d = 0.088388347648318440550;  // 1/sqrt(128), fp64
constexpr uint32_t kNegZeroBits = 0x80000000u;          // fp32 -0

__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);  // RNE
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

// fp64 -> fp32 rounded to odd: the 29 low mantissa bits an fp32 drops are
// cleared, and the lowest kept bit is set when any of them was set (their
// sum with 0x1FFFFFFF carries into bit 29 exactly then). The fp32 conversion
// of the result is exact, so it is the truncated value with its last bit
// forced to 1 when anything was dropped. This holds for |d| in the fp32
// normal range; below it the result is a subnormal fp32 or zero, which fp16
// rounds to a signed zero either way, and above it both give an infinity.
// Inf and NaN pass through (a NaN keeps a nonzero mantissa).
__device__ __forceinline__ float f64_to_f32_odd(double d) {
  const uint64_t u = __builtin_bit_cast(uint64_t, d);
  const uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
  const uint32_t sticky = ((lo & 0x1FFFFFFFu) + 0x1FFFFFFFu) & 0x20000000u;
  const uint32_t lo2 = (lo & 0xE0000000u) | sticky;
  return (float)__builtin_bit_cast(double, ((uint64_t)hi << 32) | lo2);
}

// Two fp64 values -> two fp16 (a in the low half), each rounded to nearest
// even: round to odd into fp32 first, then to nearest at 11 bits. Rounding
// to odd at 24 bits and then to nearest at 11 gives the correctly rounded
// result (Boldo and Melquiond, "Emulation of FMA and correctly rounded sums:
// proved algorithms using rounding to odd", 2008: the intermediate precision
// exceeds the final one by at least two bits). The last step is one packed
// conversion.
__device__ __forceinline__ uint32_t f64x2_to_f16x2_bits(double a, double b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 f = {f64_to_f32_odd(a), f64_to_f32_odd(b)};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
}

// x * s exactly (x an fp32, s the low or, with HI, the high fp16 half of a
// dword) as one mixed-precision FMA: the fp16 operand is widened exactly,
// the product of an fp16 and an fp16- or bf16-valued fp32 fits in 24 bits,
// and the addend -0 (negz holds its bits) leaves every product, a zero's
// sign included, unchanged.
// x * s exactly for two fp16 operands taken from the same half (HI) of the
// dwords x2 and s2: the same FMA with both operands widened in the unit.
template <bool HI>
__device__ __forceinline__ float mul_f16_by_f16(uint32_t x2, uint32_t s2, uint32_t negz) {
  float r;
  if constexpr (HI)
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,1,0] op_sel_hi:[1,1,0]"
        : "=v"(r) : "v"(x2), "v"(s2), "s"(negz));
  else
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[1,1,0]" : "=v"(r) : "v"(x2), "v"(s2), "s"(negz));
  return r;
}

template <bool HI>
__device__ __forceinline__ float mul_f32_by_f16(float x, uint32_t s2, uint32_t negz) {
  float r;
  if constexpr (HI)
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,1,0] op_sel_hi:[0,1,0]"
        : "=v"(r) : "v"(x), "v"(s2), "s"(negz));
  else
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[0,1,0]" : "=v"(r) : "v"(x), "v"(s2), "s"(negz));
  return r;
}

// bfloat16 = the upper 16 bits of an fp32, rounded to nearest even (add
// 0x7FFF plus the lowest kept bit, then truncate); a NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}
// A 16-bit output value: bf16 or fp16, both round to nearest even.
__device__ __forceinline__ uint16_t f32_to_out16(float x, int bf16) {
  return bf16 ? f32_to_bf16_bits(x) : f32_to_f16_bits(x);
}

}  // namespace exl3
