// Device-side definitions shared by the gfx950 kernels of libpagedkv.
//
// Page layout (one page = one (block, KV head) = 16 tokens x 128 dims, 2048
// two-byte elements; a block of 16 tokens of one head holds 2048 elements as on
// page "vLLM 深度解析：以 PagedAttention 与内核生态构建高吞吐 LLM 推理引擎", §2.1).
// The element order inside a page is this library's own, chosen so that a
// 64-lane wave reads a page as four contiguous 1 KiB loads of 16 bytes per lane
// and each lane's 16 bytes are directly a matrix-core operand fragment:
//
//   K: offset(t, d) = (d/8)*128 + t*8 + d%8
//      load i, lane l -> token l%16, dims 8*(4i + l/16) .. +8
//      (the A operand of v_mfma_f32_16x16x32_{f16,bf16} with rows = tokens)
//   V: offset(t, d) = ((d/16)/2)*512 + (16*(t/4) + d%16)*8 + ((d/16)%2)*4 + t%4
//      load p, lane l, element e -> token 4*(l/16) + e%4, dim 16*(2p + e/4) + l%16
//      (two B operands of v_mfma_f32_16x16x16_{f16,bf16}, k = tokens)

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kBlockSize = 16;
constexpr int kHeadSize = 128;
constexpr int kPageElems = kBlockSize * kHeadSize;  // 2048
constexpr int kWave = 64;
constexpr int kWavesPerGroup = 4;                   // decode work-groups: 4 independent waves
constexpr int kNumXcd = 8;                          // MI355X: 8 XCDs, work-groups dealt round-robin
constexpr int kMaxPartitions = 4096;                // segments per row (reduce kernel LDS bound)
constexpr int kMaxSegmentBlocks = 256;             // segment length bound (4096 tokens)
constexpr float kMaskedLogit = -__builtin_inff();
constexpr float kInitMax = -1.0e30f;                // finite: exp2(kInitMax - kInitMax) == 1

__host__ __device__ inline int k_page_offset(int t, int d) { return (d >> 3) * 128 + t * 8 + (d & 7); }

__host__ __device__ inline int v_page_offset(int t, int d) {
  const int j = d >> 4, c = d & 15, grp = t >> 2, i = t & 3;
  return (j >> 1) * 512 + (16 * grp + c) * 8 + (j & 1) * 4 + i;
}

// fp8 (E4M3) pages: 16 tokens x 128 dims of one byte, 2 KiB.  A wave reads a
// page as two contiguous 1 KiB loads of 16 bytes per lane, and lane l's 16
// bytes of load i, widened to 16-bit values, are exactly its two 16-byte
// fragments 2i and 2i+1 of the 16-bit layout above (byte order = element
// order), so the same matrix-core and dot-product code consumes them:
//   K: byte (d/64)*1024 + (16*((d/8)%4) + t)*16 + ((d/32)%2)*8 + d%8
//   V: byte (d/64)*1024 + (16*(t/4) + d%16)*16 + ((d/32)%2)*8 + ((d/16)%2)*4 + t%4
constexpr int kPageBytesFp8 = kPageElems;  // 2048
__host__ __device__ inline int k_page_offset_fp8(int t, int d) {
  return (d >> 6) * 1024 + (16 * ((d >> 3) & 3) + t) * 16 + ((d >> 5) & 1) * 8 + (d & 7);
}
__host__ __device__ inline int v_page_offset_fp8(int t, int d) {
  return (d >> 6) * 1024 + (16 * (t >> 2) + (d & 15)) * 16 + ((d >> 5) & 1) * 8 + ((d >> 4) & 1) * 4 + (t & 3);
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf168_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Element-type traits.  Storage is 16-bit words; arithmetic is fp32.
// ---------------------------------------------------------------------------
struct F16 {
  static constexpr int kMhaWavesPerSimd = 5;  // MHA decode fits 5 waves per SIMD (<= 102 VGPRs)
  // two E4M3 codes (bytes 2*hi, 2*hi+1 of w) -> two fp16 values, exact
  template <bool kHi>
  __device__ static inline uint32_t from_e4m3x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, kHi));
  }
  __device__ static inline float lo(uint32_t w) { return (float)__builtin_bit_cast(half2_t, w)[0]; }
  __device__ static inline float hi(uint32_t w) { return (float)__builtin_bit_cast(half2_t, w)[1]; }
  __device__ static inline float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c, false);
  }
  __device__ static inline uint16_t from_f32(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }
  __device__ static inline float round(float x) { return (float)(_Float16)x; }
  __device__ static inline uint32_t pack2(float a, float b) {
    half2_t h = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, h);
  }
  __device__ static inline float4_t mfma_qk(uint4 a, uint4 b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c,
                                                  0, 0, 0);
  }
  __device__ static inline float4_t mfma_pv(uint2 a, uint2 b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4_t, a), __builtin_bit_cast(half4_t, b), c,
                                                 0, 0, 0);
  }
  // the same product over 8 tokens per lane (two V fragments side by side)
  __device__ static inline float4_t mfma_pv32(uint4 a, uint4 b, float4_t c) { return mfma_qk(a, b, c); }
};

struct BF16 {
  static constexpr int kMhaWavesPerSimd = 4;  // the bf16 widening needs more registers
  template <bool kHi>
  __device__ static inline uint32_t from_e4m3x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHi));
  }
  __device__ static inline float lo(uint32_t w) { return __uint_as_float(w << 16); }
  __device__ static inline float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
  __device__ static inline float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, a), __builtin_bit_cast(bf162_t, b), c, false);
  }
  __device__ static inline uint16_t from_f32(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
  __device__ static inline float round(float x) { return (float)(__bf16)x; }
  __device__ static inline uint32_t pack2(float a, float b) {
    bf162_t h = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, h);
  }
  __device__ static inline float4_t mfma_qk(uint4 a, uint4 b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf168_t, a), __builtin_bit_cast(bf168_t, b), c,
                                                   0, 0, 0);
  }
  __device__ static inline float4_t mfma_pv(uint2 a, uint2 b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4_t, a), __builtin_bit_cast(short4_t, b),
                                                     c, 0, 0, 0);
  }
  __device__ static inline float4_t mfma_pv32(uint4 a, uint4 b, float4_t c) { return mfma_qk(a, b, c); }
};

template <class DT>
__device__ inline float dot8(uint4 a, uint4 b, float c) {
  c = DT::dot2(a.x, b.x, c);
  c = DT::dot2(a.y, b.y, c);
  c = DT::dot2(a.z, b.z, c);
  c = DT::dot2(a.w, b.w, c);
  return c;
}

// element e (0..7) of an 8 x 16-bit vector held in a uint4, as fp32
template <class DT>
__device__ inline float elem(const uint4& v, int e) {
  const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
  return (e & 1) ? DT::hi(w) : DT::lo(w);
}

// ---------------------------------------------------------------------------
// Cross-lane helpers (wave64).
// ---------------------------------------------------------------------------
template <int kCtrl>
__device__ inline float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), kCtrl, 0xf, 0xf, false));
}
constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

// max / sum over the 16 lanes of each row, result in every lane of the row
__device__ inline float row_max16(float x) {
  x = fmaxf(x, dpp<kDppQuadXor1>(x));
  x = fmaxf(x, dpp<kDppQuadXor2>(x));
  x = fmaxf(x, dpp<kDppRowHalfMirror>(x));
  x = fmaxf(x, dpp<kDppRowMirror>(x));
  return x;
}
__device__ inline float row_sum16(float x) {
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppRowHalfMirror>(x);
  x += dpp<kDppRowMirror>(x);
  return x;
}

__device__ inline float lane_from(float x, int src_lane) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src_lane << 2, __float_as_int(x)));
}

// sum / max over the 4 rows (lanes l, l^16, l^32, l^48), result in every lane.
// gfx950's row-swap permutes do the two exchanges in the vector ALU: with both
// operands x, v_permlane16_swap leaves (rows 0,0,2,2) in one result and (rows
// 1,1,3,3) in the other, so combining them pairs lane l with l^16;
// v_permlane32_swap does the same for the two halves (l with l^32).  The
// pairing, and so every rounded sum, is that of the shuffle form
// (x + x^16) + (x^32 + x^48); shuffles by lane would go through LDS.
__device__ inline float cross_row_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ inline float cross_row_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Buffer descriptor covering one 4 KiB page (gfx9 descriptor word 3:
// 32-bit data format, no swizzle); reads past the page return 0.
constexpr int kBufferDword3 = 0x00020000;
__device__ inline __amdgpu_buffer_rsrc_t page_rsrc(const uint16_t* page) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(page), 0, kPageElems * 2, kBufferDword3);
}
typedef int int4_t __attribute__((ext_vector_type(4)));
typedef int int2_t __attribute__((ext_vector_type(2)));
// Cache-policy operand of the gfx950 buffer loads: 0 is the default policy,
// kNonTemporal sets the instruction's nt bit (streaming data, not expected to
// be reused).
constexpr int kDefaultPolicy = 0;
constexpr int kNonTemporal = 2;
// 16 bytes at lane_off + kConstOff of the descriptor's range (the constant goes
// to the instruction's immediate offset, the lane part to one VGPR)
template <int kConstOff, int kPolicy = kDefaultPolicy>
__device__ inline uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t lane_off) {
  return __builtin_bit_cast(uint4,
                            __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(lane_off), kConstOff, kPolicy));
}

// Buffer descriptor covering n bytes starting at p.
__device__ inline __amdgpu_buffer_rsrc_t range_rsrc(const void* p, int n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, n, kBufferDword3);
}

// Stores through a page descriptor, at a byte offset inside the page.
template <int kPolicy = kDefaultPolicy>
__device__ inline void store16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, uint4 x) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(int4_t, x), r, static_cast<int>(byte_off), 0, kPolicy);
}
template <int kPolicy = kDefaultPolicy>
__device__ inline void store2(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, uint16_t x) {
  __builtin_amdgcn_raw_buffer_store_b16(x, r, static_cast<int>(byte_off), 0, kPolicy);
}

template <int kPolicy = kDefaultPolicy>
__device__ inline void store8(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, uint2 x) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(int2_t, x), r, static_cast<int>(byte_off), 0, kPolicy);
}
template <int kPolicy = kDefaultPolicy>
__device__ inline void store1(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, uint8_t x) {
  __builtin_amdgcn_raw_buffer_store_b8(x, r, static_cast<int>(byte_off), 0, kPolicy);
}

// E4M3 code of a float (OCP 8-bit floating point: 1 sign, 4 exponent bits with
// bias 7, 3 mantissa bits, subnormals m/8 * 2^-6, no infinities, S.1111.111 =
// NaN, largest finite 448): the nearest value, ties to the even mantissa;
// magnitudes of 448 and beyond (infinity included) give +-448, NaN gives a NaN
// code, and the sign of zero is kept.  Written from the format's definition:
// the subnormal range is a grid of step 2^-9 (rounded with the float unit's
// round-to-nearest-even), the normal range keeps 3 of the 23 mantissa bits.
__device__ inline uint32_t e4m3_encode(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t au = u & 0x7FFFFFFFu;
  if (au > 0x7F800000u) return sign | 0x7Fu;  // NaN
  if (au >= 0x43E00000u) return sign | 0x7Eu;  // |x| >= 448
  if (au < 0x3C800000u) {                      // |x| < 2^-6: multiples of 2^-9
    // exact scaling; values below 2^-126 read as zero here and round to 0 anyway
    const float grid = __uint_as_float(au) * 512.0f;
    return sign | static_cast<uint32_t>(__builtin_rintf(grid));  // 8 is the code of 2^-6
  }
  const uint32_t mant = au & 0x7FFFFFu;
  uint32_t q = (((au >> 23) - 120u) << 3) | (mant >> 20);  // exponent bias 127 -> 7
  const uint32_t rem = mant & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ++q;  // a mantissa carry bumps the exponent
  return sign | (q > 0x7Eu ? 0x7Eu : q);
}

__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline int wave_id_uniform() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

}  // namespace pkv
