// Device helpers shared by the libdpnorm kernels (gfx950 / CDNA4).
//
// MFMA operand conventions used throughout (v_mfma_f32_16x16x32_bf16):
//   A operand: lane l supplies 8 bf16 of row (l % 16) at K slots 8*(l/16)+j
//   B operand: lane l supplies 8 bf16 of column (l % 16) at K slots 8*(l/16)+j
//   C/D      : lane l holds rows 4*(l/16) + r, r = 0..3, of column (l % 16)
// and for v_mfma_f32_16x16x4f32 one fp32 value per lane at K slot (l/16), with
// the same C/D layout. (v_mfma_f64_16x16x4f64 differs: lane l holds rows
// l/16 + 4 r, r = 0..3, of column l % 16.)
// Only the pairing of A and B K slots matters for a contraction, so the
// kernels are free to map any contraction index to a (group, element) slot
// as long as both operands use the same map.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dpn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Round-to-nearest-even float -> bf16 bit pattern (NaN kept a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Split x into hi + lo, both bf16, with |x - hi - lo| <= 2^-17 |x| (x - hi is
// exact in fp32 because hi is within a factor of two of x).
__device__ __forceinline__ void split_bf16(float x, uint32_t& hi, uint32_t& lo) {
  hi = f32_to_bf16_bits(x);
  lo = f32_to_bf16_bits(x - bf16_bits_to_f32(hi));
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ f32x4_t mfma_bf16(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma_f32(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Global-memory accesses through the global address space. Pointers that a
// kernel reads from a device-side record are generic to the compiler, which
// would emit flat instructions; flat loads may alias LDS, so the compiler
// would then wait for every outstanding direct-to-LDS load before each one.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
#define DPN_GLOBAL __attribute__((address_space(1)))
__device__ __forceinline__ uint4 ldg16(const void* p) {
  const u32x4_t v = *(const DPN_GLOBAL u32x4_t*)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 ldg16_stream(const void* p) {  // non-temporal: streamed past the caches
  const u32x4_t v = __builtin_nontemporal_load((const DPN_GLOBAL u32x4_t*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float ldg_f32(const void* p) { return *(const DPN_GLOBAL float*)p; }
__device__ __forceinline__ float4 ldg_f32x4(const void* p) {
  const f32x4_t v = *(const DPN_GLOBAL f32x4_t*)p;
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void stg16(void* p, const uint4& v) { *(DPN_GLOBAL u32x4_t*)p = u32x4_t{v.x, v.y, v.z, v.w}; }
__device__ __forceinline__ void stg_f32(void* p, float v) { *(DPN_GLOBAL float*)p = v; }

__device__ __forceinline__ uint4 pack8(const uint32_t b[8]) {
  return make_uint4(b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16), b[6] | (b[7] << 16));
}

// In-register transpose of an 8 x 8 block of bf16.
// in[s] holds 8 consecutive elements (columns e = 0..7) of row s;
// out[e] holds rows s = 0..7 of column e, row 0 in the low half of word 0.
// Low halves (pack_lo16) or high halves (pack_hi16) of a and b as one word,
// a's half in the low 16 bits: one v_perm_b32 each, whose result byte i is
// byte sel_i of the eight bytes {a (0-3), b (4-7)}.
__device__ __forceinline__ uint32_t pack_lo16(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }
__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}
__device__ __forceinline__ void transpose8x8_bf16(const uint4 in[8], uint4 out[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int w = e >> 1;
    uint32_t q[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t a = word(in[2 * j], w), b = word(in[2 * j + 1], w);
      q[j] = (e & 1) ? pack_hi16(a, b) : pack_lo16(a, b);
    }
    out[e] = make_uint4(q[0], q[1], q[2], q[3]);
  }
}

// Row of a 32-row chunk that K slot (group g, element s) of a bf16 MFMA
// operand stands for. It is chosen so that the rows a lane holds in the
// accumulators of two stacked 16 x 16 tiles (rows 4g + r and 16 + 4g + r)
// are exactly the rows of its K slots: a stage-1 result feeds stage 2 from
// the lane's own registers.
__device__ __forceinline__ int slot_row(int g, int s) { return 16 * (s >> 2) + 4 * g + (s & 3); }

// One DPP move of a double (both 32-bit halves); lanes whose source lies
// outside their row, or whose row is masked off, receive 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint2 h = __builtin_bit_cast(uint2, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)h.x, CTRL, ROW_MASK, 0xf, true);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)h.y, CTRL, ROW_MASK, 0xf, true);
  return __builtin_bit_cast(double, make_uint2(lo, hi));
}

// Sum over the 64 lanes, the same in every lane, in a fixed order: inclusive
// prefix sums within each row of 16 lanes (DPP row_shr 1, 2, 4, 8), then
// lane 15 of rows 0 and 2 added into rows 1 and 3 (row_bcast:15) and lane 31
// into rows 2 and 3 (row_bcast:31), so lane 63 holds the total.
__device__ __forceinline__ double wave_sum(double v) {
  v += dpp_f64<0x111, 0xf>(v);   // row_shr:1
  v += dpp_f64<0x112, 0xf>(v);   // row_shr:2
  v += dpp_f64<0x114, 0xf>(v);   // row_shr:4
  v += dpp_f64<0x118, 0xf>(v);   // row_shr:8
  v += dpp_f64<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
  v += dpp_f64<0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3
  const uint2 h = __builtin_bit_cast(uint2, v);
  return __builtin_bit_cast(double, make_uint2((uint32_t)__builtin_amdgcn_readlane((int)h.x, 63),
                                               (uint32_t)__builtin_amdgcn_readlane((int)h.y, 63)));
}

// Map a linear block index to a work item so that each XCD (blocks are
// dispatched round-robin over the 8 XCDs) walks one contiguous range of the
// item list; neighbouring items then share their XCD's L2.
__device__ __forceinline__ int xcd_item(uint32_t b, uint32_t n) {
  const uint32_t x = b & 7u, j = b >> 3;
  const uint32_t per = n >> 3, rem = n & 7u;
  return (int)(x * per + (x < rem ? x : rem) + j);
}

// ---------------------------------------------------------------------------
// Direct global-to-LDS streaming (global_load_lds_dwordx4), shared by the
// stage kernels, the exact comparator and the calibration stream.
// ---------------------------------------------------------------------------
// s_waitcnt with only the vector-memory counter limited (expcnt, lgkmcnt at max).
#define DPN_WAIT_VMCNT(N) __builtin_amdgcn_s_waitcnt(((N) & 15) | (7 << 4) | (15 << 8) | ((((N) >> 4) & 3) << 14))

// 16 bytes per lane from global memory to LDS at lds_addr + 16 * lane
// (lds_addr wave-uniform), non-temporal (dma16_stream) or cached (dma16).
// The loads are issued from inline assembly so that the compiler adds no
// waits for them: the kernels place their own vector-memory waits. M0
// carries the LDS address; nothing else in these kernels uses M0.
__device__ __forceinline__ void dma16_stream(const void* src, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src),
               "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory");
}
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src),
               "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory");
}
// Same, past this CU's L1 (sc0): the data comes from the XCD's L2, where
// another CU of the same XCD has just stored it.
__device__ __forceinline__ void dma16_l2(const void* src, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off sc0" ::"v"(src),
               "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory");
}
// A 32-bit counter read with a returning atomic add of 0: performed where
// the counter's atomic increments are (written out because the compiler
// would turn an atomic add of 0 into a load, and atomic loads skip the L2
// that holds the increments), then waited for.
__device__ __forceinline__ uint32_t atomic_read_u32(uint32_t* p) {
  uint32_t v;
  const uint32_t zero = 0u;
  asm volatile("global_atomic_add %0, %1, %2, off sc0\n\ts_waitcnt vmcnt(0)" : "=&v"(v) : "v"(p), "v"(zero) : "memory");
  return v;
}
// Two doubles read past this CU's L1 (sc0), both loads in flight, then waited for.
__device__ __forceinline__ void ldg2_f64_l2(const double* p0, const double* p1, double& a, double& b) {
  asm volatile("global_load_dwordx2 %0, %2, off sc0\n\tglobal_load_dwordx2 %1, %3, off sc0\n\ts_waitcnt vmcnt(0)"
               : "=&v"(a), "=&v"(b)
               : "v"(p0), "v"(p1)
               : "memory");
}
// Work-group barrier that the compiler may not move memory accesses across.
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt vmcnt(after * P) for after in 0..2: at most `after` later
// stages' loads (P per stage) still outstanding.
template <int P>
__device__ __forceinline__ void wait_after(int after) {
  if (after >= 2) DPN_WAIT_VMCNT(2 * P);
  else if (after == 1) DPN_WAIT_VMCNT(P);
  else DPN_WAIT_VMCNT(0);
}

// Transposing LDS read (ds_read_b64_tr_b16). Within each group of 16 lanes,
// lane 4 j + q supplies the address of 4 consecutive 16-bit elements; lane i
// of the group receives element i % 4 of the data of lane 4 j + i / 4, for
// j = 0..3. Pointing lane 4 j + q at row k0 + j, columns m0 + 4 q .. + 3 of a
// row-major bf16 block gives lane i rows k0 .. k0 + 3 of column m0 + i: half
// of a 16 x 32 MFMA operand (K along rows) with no register transpose.
typedef short bf16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16(const unsigned char* p) {
  const bf16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) bf16x4_t*)
                                                                 (__attribute__((address_space(3))) void*)p);
  return __builtin_bit_cast(uint2, v);
}

}  // namespace dpn
