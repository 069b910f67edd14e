// Device helpers shared by the gfx950 kernels: cross-lane exchanges for the
// 32-wide Walsh-Hadamard butterfly, nibble unpacking, int8 dot products and
// loads.  Wave64 throughout.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#define SVG_DEV __device__ __forceinline__

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef unsigned u32;

// ------------------------------------------------------- lane exchanges
// xor-1 and xor-2 within a quad: DPP quad_perm; xor-4/8/16 within 32 lanes:
// ds_swizzle in bit-mask mode (and=0x1f, xor=mask); xor-32: ds_bpermute.
SVG_DEV int lane_xor1(int v) { return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, true); }
SVG_DEV int lane_xor2(int v) { return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, true); }
SVG_DEV int lane_xor4(int v) { return __builtin_amdgcn_ds_swizzle(v, 0x1F | (4 << 10)); }
SVG_DEV int lane_xor8(int v) { return __builtin_amdgcn_ds_swizzle(v, 0x1F | (8 << 10)); }
SVG_DEV int lane_xor16(int v) { return __builtin_amdgcn_ds_swizzle(v, 0x1F | (16 << 10)); }
SVG_DEV int lane_xor32(int v) {
  const int lane = __lane_id();
  return __builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, v);
}

template <int MASK>
SVG_DEV int lane_xor(int v) {
  if constexpr (MASK == 1) return lane_xor1(v);
  else if constexpr (MASK == 2) return lane_xor2(v);
  else if constexpr (MASK == 4) return lane_xor4(v);
  else if constexpr (MASK == 8) return lane_xor8(v);
  else if constexpr (MASK == 16) return lane_xor16(v);
  else return lane_xor32(v);
}
template <int MASK>
SVG_DEV float lane_xorf(float v) { return __int_as_float(lane_xor<MASK>(__float_as_int(v))); }

// Maximum over the wave, the same in every lane, with no LDS access: DPP
// inside each quad and each row of 16 lanes (row rotations by 4 and 8), then
// the four rows' values read out as scalars.  Exact (max is order-free).
SVG_DEV float wave_max(float v) {
  v = fmaxf(v, lane_xorf<1>(v));
  v = fmaxf(v, lane_xorf<2>(v));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false)));
  const int b = __float_as_int(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(b, 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(b, 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(b, 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(b, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// ------------------------------------------- 32-wide Walsh-Hadamard butterfly
// A block of 32 values is spread over 8 consecutive lanes, 4 consecutive
// values per lane (lane j of the block holds elements 4j..4j+3).  Stages run
// h = 1, 2 inside the lane, then h = 4, 8, 16 across lanes j^1, j^2, j^4.  At
// every stage the lower element of a pair becomes (a + b) and the upper one
// (a - b): one rounded fp32 operation each, in ascending stage order.
#pragma clang fp contract(off)
SVG_DEV void fwht32_lane4(float& e0, float& e1, float& e2, float& e3) {
  const int j = __lane_id() & 7;
  float a0 = e0 + e1, a1 = e0 - e1, a2 = e2 + e3, a3 = e2 - e3;  // h = 1
  e0 = a0 + a2; e2 = a0 - a2; e1 = a1 + a3; e3 = a1 - a3;        // h = 2
  {
    float p0 = lane_xorf<1>(e0), p1 = lane_xorf<1>(e1), p2 = lane_xorf<1>(e2), p3 = lane_xorf<1>(e3);
    const bool up = j & 1;                                         // h = 4
    e0 = up ? p0 - e0 : e0 + p0; e1 = up ? p1 - e1 : e1 + p1;
    e2 = up ? p2 - e2 : e2 + p2; e3 = up ? p3 - e3 : e3 + p3;
  }
  {
    float p0 = lane_xorf<2>(e0), p1 = lane_xorf<2>(e1), p2 = lane_xorf<2>(e2), p3 = lane_xorf<2>(e3);
    const bool up = j & 2;                                         // h = 8
    e0 = up ? p0 - e0 : e0 + p0; e1 = up ? p1 - e1 : e1 + p1;
    e2 = up ? p2 - e2 : e2 + p2; e3 = up ? p3 - e3 : e3 + p3;
  }
  {
    float p0 = lane_xorf<4>(e0), p1 = lane_xorf<4>(e1), p2 = lane_xorf<4>(e2), p3 = lane_xorf<4>(e3);
    const bool up = j & 4;                                         // h = 16
    e0 = up ? p0 - e0 : e0 + p0; e1 = up ? p1 - e1 : e1 + p1;
    e2 = up ? p2 - e2 : e2 + p2; e3 = up ? p3 - e3 : e3 + p3;
  }
}

// Transform block B = 32 or 64 (the wave-wide variant).  A 64-block spans 16
// consecutive lanes: the 32-wide butterfly runs on each half (lanes j and
// j ^ 8 hold elements i and i + 32), then the stage h = 32 pairs them, the
// lower element becoming (a + b) and the upper one (a - b) as at every stage.
template <int B>
SVG_DEV void fwht_lane4(float& e0, float& e1, float& e2, float& e3) {
  static_assert(B == 32 || B == 64, "transform block 32 or 64");
  fwht32_lane4(e0, e1, e2, e3);
  if constexpr (B == 64) {
    const float p0 = lane_xorf<8>(e0), p1 = lane_xorf<8>(e1), p2 = lane_xorf<8>(e2), p3 = lane_xorf<8>(e3);
    const bool up = __lane_id() & 8;                               // h = 32
    e0 = up ? p0 - e0 : e0 + p0; e1 = up ? p1 - e1 : e1 + p1;
    e2 = up ? p2 - e2 : e2 + p2; e3 = up ? p3 - e3 : e3 + p3;
  }
}

// Sign flip of four values by four packed int8 signs (+1 / -1): exact.
SVG_DEV void apply_signs4(float& e0, float& e1, float& e2, float& e3, int packed) {
  e0 = e0 * (float)(int8_t)(packed & 0xFF);
  e1 = e1 * (float)(int8_t)((packed >> 8) & 0xFF);
  e2 = e2 * (float)(int8_t)((packed >> 16) & 0xFF);
  e3 = e3 * (float)(int8_t)((packed >> 24) & 0xFF);
}

// --------------------------------------------------------------- integers
// Packed word of 8 nibbles (k = 0..7, nibble i at bits 4i) -> two int8x4
// words: even-k codes {0,2,4,6} and odd-k codes {1,3,5,7}.
SVG_DEV u32 nib_even(u32 w) { return w & 0x0F0F0F0Fu; }
SVG_DEV u32 nib_odd(u32 w) { return (w >> 4) & 0x0F0F0F0Fu; }
// The matching reorder of 8 int8 activation codes held in two words
// (a0 = k 0..3, a1 = k 4..7): even-k bytes and odd-k bytes.
SVG_DEV u32 act_even(u32 a0, u32 a1) { return __builtin_amdgcn_perm(a1, a0, 0x06040200u); }
SVG_DEV u32 act_odd(u32 a0, u32 a1) { return __builtin_amdgcn_perm(a1, a0, 0x07050301u); }

SVG_DEV int dot4(u32 a, u32 b, int c) { return __builtin_amdgcn_sdot4((int)a, (int)b, c, false); }

// ------------------------------------------------------------------ loads
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
SVG_DEV uint4 load_nt16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
SVG_DEV uint4 load16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

SVG_DEV float half_bits_to_float(uint16_t h) { return __half2float(__ushort_as_half(h)); }

// Raw buffer loads.  A buffer resource covers [base, base + nbytes); a load
// whose offset lies outside returns zeros instead of faulting, which makes
// ragged tails branch-free: an out-of-range lane passes kOOB as its offset.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr u32 kOOB = 0x80000000u;      // beyond every buffer this library builds
constexpr int kNT = 2;                 // cache policy: non-temporal (streamed once)
constexpr int kSC1 = 16;               // cache policy: device scope (sc1: past the caches of one XCC)
SVG_DEV rsrc_t make_rsrc(const void* base, u32 nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)nbytes, 0x00020000);
}
SVG_DEV u32x4 bload16(rsrc_t r, u32 off) { return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0); }
SVG_DEV u32x4 bload16_nt(rsrc_t r, u32 off) { return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNT); }
template <int AUX>
SVG_DEV u32x4 bload16a(rsrc_t r, u32 off) { return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX); }
SVG_DEV u32 bload4(rsrc_t r, u32 off) { return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0); }
SVG_DEV uint16_t bload2(rsrc_t r, u32 off) { return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0); }
SVG_DEV uint8_t bload1(rsrc_t r, u32 off) { return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0); }

// NB contiguous bytes (NB in 1, 2, 4, 8, 16, 32) from an NB-aligned offset
// (16-aligned for 32), as little-endian 32-bit words.
template <int NB>
struct Bytes {
  u32 w[NB >= 4 ? NB / 4 : 1];
};
template <int NB>
SVG_DEV void bload_bytes(Bytes<NB>& o, rsrc_t r, u32 off) {
  if constexpr (NB == 32) {
    const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16u, 0, 0);
    for (int i = 0; i < 4; ++i) { o.w[i] = a[i]; o.w[4 + i] = b[i]; }
  } else if constexpr (NB == 16) {
    const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    for (int i = 0; i < 4; ++i) o.w[i] = a[i];
  } else if constexpr (NB == 8) {
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 a = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    o.w[0] = a[0];
    o.w[1] = a[1];
  } else if constexpr (NB == 4) {
    o.w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  } else if constexpr (NB == 2) {
    o.w[0] = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
  } else {
    o.w[0] = __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
  }
}
// The i-th fp16 of a block of words, as float.
SVG_DEV float half_at(const u32* w, int i) {
  return half_bits_to_float((uint16_t)((i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFF)));
}
// The i-th 4-bit value of a block of words.
SVG_DEV int nibble_at(const u32* w, int i) { return (int)((w[i >> 3] >> (4 * (i & 7))) & 0xF); }
