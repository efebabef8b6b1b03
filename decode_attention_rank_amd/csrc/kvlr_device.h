// Device helpers shared by the kvlr kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace kvlr {

constexpr int kWave = 64;

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Streaming loads: marked non-temporal, for data read once per launch.
__device__ inline uint4 load16_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ inline uint2 load8_stream(const void* p) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(v.x, v.y);
}

// Storage policies. A chunk holds CH elements in CB bytes: 8 bf16 or 4 f32
// in 16 bytes, or 8 FP8 latents in 8 bytes. Raw is the chunk as loaded.
struct BF16 {
  static constexpr int CH = 8;
  static constexpr int ELEM_BYTES = 2;
  static constexpr int CB = 16;
  using Raw = uint4;
  __device__ static inline Raw load_stream(const void* p) { return load16_stream(p); }
  __device__ static inline bf16x8 to_bf16x8(const Raw& r) { return __builtin_bit_cast(bf16x8, r); }
  // 16 loaded bytes hold one token's chunk: fragment h = 0 only
  __device__ static inline bf16x8 frag_of16(const uint4& r, int) { return __builtin_bit_cast(bf16x8, r); }
  // element e of a chunk as float (bf16 -> f32 is a 16-bit shift, exact)
  __device__ static inline void unpack(const uint4& c, float (&x)[CH]) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static inline float load1(const void* base, long idx) {
    const uint16_t u = reinterpret_cast<const uint16_t*>(base)[idx];
    return __uint_as_float(static_cast<uint32_t>(u) << 16);
  }
  // elements idx .. idx+3 (idx a multiple of 4) in one 8-byte read
  __device__ static inline void load4(const void* base, long idx, float (&x)[4]) {
    const uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(base) + idx);
    x[0] = __uint_as_float(w.x << 16);
    x[1] = __uint_as_float(w.x & 0xffff0000u);
    x[2] = __uint_as_float(w.y << 16);
    x[3] = __uint_as_float(w.y & 0xffff0000u);
  }
};

struct F32 {
  static constexpr int CH = 4;
  static constexpr int ELEM_BYTES = 4;
  static constexpr int CB = 16;
  using Raw = uint4;
  __device__ static inline Raw load_stream(const void* p) { return load16_stream(p); }
  __device__ static inline void unpack(const uint4& c, float (&x)[CH]) {
    x[0] = __uint_as_float(c.x);
    x[1] = __uint_as_float(c.y);
    x[2] = __uint_as_float(c.z);
    x[3] = __uint_as_float(c.w);
  }
  __device__ static inline float load1(const void* base, long idx) {
    return reinterpret_cast<const float*>(base)[idx];
  }
  __device__ static inline void load4(const void* base, long idx, float (&x)[4]) {
    const float4 w = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + idx);
    x[0] = w.x;
    x[1] = w.y;
    x[2] = w.z;
    x[3] = w.w;
  }
};

// Two E4M3 codes (bytes 0,1 of w, or bytes 2,3 with HI) to two bf16 in one
// instruction, with scale 1 (exact: every E4M3 value is a bf16). Written as
// assembly because the compiler's builtin for it is followed by a permute
// that copies the first element into both halves; checked on all 256 codes
// in each byte position against the float32 decode.
template <bool HI>
__device__ inline uint32_t fp8x2_to_bf16x2(uint32_t w) {
  uint32_t r;
  if (HI)
    asm("v_cvt_scalef32_pk_bf16_fp8 %0, %1, 1.0 op_sel:[1,0,0]" : "=v"(r) : "v"(w));
  else
    asm("v_cvt_scalef32_pk_bf16_fp8 %0, %1, 1.0" : "=v"(r) : "v"(w));
  return r;
}

// OCP 8-bit floating point E4M3 (4 exponent bits, bias 7, 3 stored
// significand bits, no infinities, largest finite value 448): latents only.
// Every E4M3 value is exact in bfloat16 and float32, so decoding is exact:
// v_cvt_pk_f32_fp8 decodes all 256 codes as OCP E4M3 on gfx950 (two per
// instruction, bytes 0,1 or 2,3 of a word); matrix-core operands take the
// codes to bf16 directly, two per instruction.
struct FP8 {
  static constexpr int CH = 8;
  static constexpr int ELEM_BYTES = 1;
  static constexpr int CB = 8;
  using Raw = uint2;
  __device__ static inline Raw load_stream(const void* p) { return load8_stream(p); }
  __device__ static inline void unpack(const Raw& r, float (&x)[CH]) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    const uint32_t w[2] = {r.x, r.y};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const f2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[i]), false);
      const f2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[i]), true);
      x[4 * i] = lo[0];
      x[4 * i + 1] = lo[1];
      x[4 * i + 2] = hi[0];
      x[4 * i + 3] = hi[1];
    }
  }
  // bytes 0..7 -> bf16 elements 0..7
  __device__ static inline bf16x8 to_bf16x8(const Raw& r) {
    return __builtin_bit_cast(bf16x8, make_uint4(fp8x2_to_bf16x2<false>(r.x), fp8x2_to_bf16x2<true>(r.x),
                                                 fp8x2_to_bf16x2<false>(r.y), fp8x2_to_bf16x2<true>(r.y)));
  }
  // 16 loaded bytes hold two tokens' chunks: fragment h of token h
  __device__ static inline bf16x8 frag_of16(const uint4& r, int h) {
    return to_bf16x8(h ? make_uint2(r.z, r.w) : make_uint2(r.x, r.y));
  }
};

// float32 -> E4M3 code, round to nearest even, saturating at +-448 (the
// converter itself maps magnitudes past 464 to NaN); NaN stays NaN.
__device__ inline uint32_t f32_to_fp8_rne_sat(float f) {
  const float c = (f != f) ? f : fminf(fmaxf(f, -448.f), 448.f);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(c, 0.f, 0, false)) & 0xffu;
}

// float32 -> bfloat16 bits, round to nearest even (NaN stays NaN).
__device__ inline uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// 8 floats as bfloat16: hi = RNE(x), lo = RNE(x - hi); hi + lo carries about
// 16 significant bits of x, so a product with a bf16 latent through the two
// halves is exact to about 2^-18 relative.
__device__ inline void split_bf16x8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t h0 = f32_to_bf16_rne(x[2 * i]), h1 = f32_to_bf16_rne(x[2 * i + 1]);
    const uint32_t l0 = f32_to_bf16_rne(x[2 * i] - __uint_as_float(h0 << 16));
    const uint32_t l1 = f32_to_bf16_rne(x[2 * i + 1] - __uint_as_float(h1 << 16));
    h[i] = h0 | (h1 << 16);
    l[i] = l0 | (l1 << 16);
  }
  hi = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
  lo = __builtin_bit_cast(bf16x8, make_uint4(l[0], l[1], l[2], l[3]));
}

// A sequence length as the kernels use it: within [0, max_pages * P], the
// tokens its page-table row can address (a longer length is a caller error
// that kvlr_check_page_tables reports; the kernels never index past the row).
__device__ inline int table_len(int L, int max_pages, int P) {
  const int cap = max_pages * P;
  return L < 0 ? 0 : (L > cap ? cap : L);
}

__device__ inline uint4 load16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

__device__ inline void store16(void* p, const uint4& v) {
  *reinterpret_cast<uint4*>(p) = v;
}


// ---------------------------------------------------------------------------
// Cross-workgroup hand-off without cache flushes.
//
// The L2 of each XCD is not coherent with the others, and a release/acquire
// fence at device scope writes back and invalidates the whole L2 of the XCD
// that runs it. Instead, values that another workgroup will read are written
// and read with device-scope relaxed atomics (coherent at device scope: they
// bypass the non-coherent L2 lines), each wave waits for its stores to
// complete, and the ticket itself is a device-scope atomic add. A workgroup
// that draws the last ticket has therefore seen every other workgroup's
// stores completed before their tickets.
__device__ inline void store_shared_f32(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float load_shared_f32(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void wait_stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ inline uint32_t take_ticket(uint32_t* counter) {
  return __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void reset_ticket(uint32_t* counter) {
  __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, class F>
__device__ inline void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// ---------------------------------------------------------------------------
// Wave-uniform operands in scalar registers.
//
// Query values are the same for every lane of a wave, so they belong in
// SGPRs where a VALU FMA reads them for free. Loading them with plain C++
// lets the compiler hoist every query value of a kernel out of its loop and
// spill the excess into VGPR lanes (one v_readlane per use). These helpers
// issue the scalar loads where they are used and wait for them inside the
// same asm block, so no load is ever in flight when the block ends.
typedef float sreg8 __attribute__((ext_vector_type(8)));
typedef float sreg4 __attribute__((ext_vector_type(4)));

template <int N>
struct SRegs;
template <>
struct SRegs<8> {
  using T = sreg8;
};
template <>
struct SRegs<4> {
  using T = sreg4;
};

#define KVLR_SL8 "s_load_dwordx8 "
#define KVLR_SL4 "s_load_dwordx4 "

// out[h] = p[h * STRIDE + OFF .. + N) for h < G (floats), N = 4 or 8.
template <int G, int N, int STRIDE, int OFF>
__device__ inline void sload_heads(const float* p, typename SRegs<N>::T (&out)[G]) {
  static_assert(N == 4 || N == 8, "chunk of 4 or 8 floats");
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group size");
  constexpr int B = 4;  // bytes per float
  if constexpr (N == 8) {
    if constexpr (G == 1) {
      asm volatile(KVLR_SL8 "%0, %1, %2\n\ts_waitcnt lgkmcnt(0)"
                   : "=s"(out[0]) : "s"(p), "i"(OFF * B));
    } else if constexpr (G == 2) {
      asm volatile(KVLR_SL8 "%0, %2, %3\n\t" KVLR_SL8 "%1, %2, %4\n\ts_waitcnt lgkmcnt(0)"
                   : "=s"(out[0]), "=s"(out[1])
                   : "s"(p), "i"(OFF * B), "i"((STRIDE + OFF) * B));
    } else if constexpr (G == 4) {
      asm volatile(KVLR_SL8 "%0, %4, %5\n\t" KVLR_SL8 "%1, %4, %6\n\t" KVLR_SL8 "%2, %4, %7\n\t"
                   KVLR_SL8 "%3, %4, %8\n\ts_waitcnt lgkmcnt(0)"
                   : "=s"(out[0]), "=s"(out[1]), "=s"(out[2]), "=s"(out[3])
                   : "s"(p), "i"(OFF * B), "i"((STRIDE + OFF) * B), "i"((2 * STRIDE + OFF) * B),
                     "i"((3 * STRIDE + OFF) * B));
    } else {
      asm volatile(KVLR_SL8 "%0, %8, %9\n\t" KVLR_SL8 "%1, %8, %10\n\t" KVLR_SL8 "%2, %8, %11\n\t"
                   KVLR_SL8 "%3, %8, %12\n\t" KVLR_SL8 "%4, %8, %13\n\t" KVLR_SL8 "%5, %8, %14\n\t"
                   KVLR_SL8 "%6, %8, %15\n\t" KVLR_SL8 "%7, %8, %16\n\ts_waitcnt lgkmcnt(0)"
                   : "=s"(out[0]), "=s"(out[1]), "=s"(out[2]), "=s"(out[3]), "=s"(out[4]),
                     "=s"(out[5]), "=s"(out[6]), "=s"(out[7])
                   : "s"(p), "i"(OFF * B), "i"((STRIDE + OFF) * B), "i"((2 * STRIDE + OFF) * B),
                     "i"((3 * STRIDE + OFF) * B), "i"((4 * STRIDE + OFF) * B),
                     "i"((5 * STRIDE + OFF) * B), "i"((6 * STRIDE + OFF) * B),
                     "i"((7 * STRIDE + OFF) * B));
    }
  } else {
    if constexpr (G == 1) {
      asm volatile(KVLR_SL4 "%0, %1, %2\n\ts_waitcnt lgkmcnt(0)"
                   : "=s"(out[0]) : "s"(p), "i"(OFF * B));
    } else if constexpr (G == 2) {
      asm volatile(KVLR_SL4 "%0, %2, %3\n\t" KVLR_SL4 "%1, %2, %4\n\ts_waitcnt lgkmcnt(0)"
                   : "=s"(out[0]), "=s"(out[1])
                   : "s"(p), "i"(OFF * B), "i"((STRIDE + OFF) * B));
    } else if constexpr (G == 4) {
      asm volatile(KVLR_SL4 "%0, %4, %5\n\t" KVLR_SL4 "%1, %4, %6\n\t" KVLR_SL4 "%2, %4, %7\n\t"
                   KVLR_SL4 "%3, %4, %8\n\ts_waitcnt lgkmcnt(0)"
                   : "=s"(out[0]), "=s"(out[1]), "=s"(out[2]), "=s"(out[3])
                   : "s"(p), "i"(OFF * B), "i"((STRIDE + OFF) * B), "i"((2 * STRIDE + OFF) * B),
                     "i"((3 * STRIDE + OFF) * B));
    } else {
      asm volatile(KVLR_SL4 "%0, %8, %9\n\t" KVLR_SL4 "%1, %8, %10\n\t" KVLR_SL4 "%2, %8, %11\n\t"
                   KVLR_SL4 "%3, %8, %12\n\t" KVLR_SL4 "%4, %8, %13\n\t" KVLR_SL4 "%5, %8, %14\n\t"
                   KVLR_SL4 "%6, %8, %15\n\t" KVLR_SL4 "%7, %8, %16\n\ts_waitcnt lgkmcnt(0)"
                   : "=s"(out[0]), "=s"(out[1]), "=s"(out[2]), "=s"(out[3]), "=s"(out[4]),
                     "=s"(out[5]), "=s"(out[6]), "=s"(out[7])
                   : "s"(p), "i"(OFF * B), "i"((STRIDE + OFF) * B), "i"((2 * STRIDE + OFF) * B),
                     "i"((3 * STRIDE + OFF) * B), "i"((4 * STRIDE + OFF) * B),
                     "i"((5 * STRIDE + OFF) * B), "i"((6 * STRIDE + OFF) * B),
                     "i"((7 * STRIDE + OFF) * B));
    }
  }
}

#undef KVLR_SL8
#undef KVLR_SL4

// acc[h] += q_h[OFF .. OFF+CH) . x for the G heads of a group, q_h = qp + h*STRIDE.
// Heads are loaded in blocks of at most 32 scalar registers. The empty asm on
// the accumulators pins a block's FMAs before the next block's loads, so the
// scheduler cannot batch every block's loads first and spill the registers.
template <int G, int CH, int STRIDE, int OFF>
__device__ inline void fma_heads(const float* qp, const float (&x)[CH], float (&acc)[G]) {
  constexpr int HB = (G * CH <= 32) ? G : 32 / CH;
  static_for<0, G / HB>([&](auto hb) {
    constexpr int H0 = decltype(hb)::value * HB;
    typename SRegs<CH>::T q[HB];
    sload_heads<HB, CH, STRIDE, H0 * STRIDE + OFF>(qp, q);
#pragma unroll
    for (int h = 0; h < HB; ++h) {
#pragma unroll
      for (int e = 0; e < CH; ++e) acc[H0 + h] = fmaf(q[h][e], x[e], acc[H0 + h]);
      asm volatile("" : "+v"(acc[H0 + h]));
    }
  });
}

// ---------------------------------------------------------------------------
// Wave-uniform operands broadcast from VGPRs.
//
// A group's projected queries (G x W floats) are spread over NQ = G*W/16
// VGPRs: lane l of register k holds q_flat[16k + (l & 15)], the same 16
// values in each 16-lane row. v_fmac_f32 with the DPP row_newbcast:n
// modifier reads lane n of its row for src0, so one VALU instruction does
// acc += q_flat[16k + n] * x for every lane with no scalar loads at all.
// The query registers are written only by global loads (never by a VALU
// just before), so the DPP source needs no extra wait states.
template <int N>
__device__ inline void fmac_bcast(float& acc, float q, float x) {
  asm volatile("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
               : "+v"(acc)
               : "v"(q), "v"(x), "n"(N));
}

template <int NQ>
__device__ inline void load_q_rows(const float* qflat, float (&qv)[NQ]) {
  const int l16 = threadIdx.x & 15;
#pragma unroll
  for (int k = 0; k < NQ; ++k) qv[k] = qflat[16 * k + l16];
}

// acc[h] += q_flat[h*STRIDE + OFF + e] * x[e] for e < CH, h < G.
template <int G, int CH, int STRIDE, int OFF, int NQ>
__device__ inline void fma_heads_bcast(const float (&qv)[NQ], const float (&x)[CH],
                                       float (&acc)[G]) {
  static_for<0, G>([&](auto hh) {
    constexpr int H = decltype(hh)::value;
    static_for<0, CH>([&](auto ee) {
      constexpr int F = H * STRIDE + OFF + decltype(ee)::value;
      fmac_bcast<F % 16>(acc[H], qv[F / 16], x[decltype(ee)::value]);
    });
  });
}

// ---------------------------------------------------------------------------
// DPP reductions (no LDS traffic). Steps within a 16-lane row use quad_perm
// and mirrors; rows are combined with row_bcast, which leaves the full
// result in lane 63.
template <int CTRL, int ROW_MASK = 0xf>
__device__ inline float dpp(float old, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL,
                                                    ROW_MASK, 0xf, false));
}

constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
constexpr int kDppBcast15 = 0x142;
constexpr int kDppBcast31 = 0x143;

// Max over each aligned 16-lane row; every lane of the row gets it.
__device__ inline float row16_max(float v) {
  v = fmaxf(v, dpp<kDppXor1>(v, v));
  v = fmaxf(v, dpp<kDppXor2>(v, v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v, v));
  v = fmaxf(v, dpp<kDppMirror>(v, v));
  return v;
}

// Max over the whole wave, returned as a wave-uniform value.
__device__ inline float wave_max_u(float v) {
  v = row16_max(v);
  v = fmaxf(v, dpp<kDppBcast15, 0xa>(-__builtin_huge_valf(), v));
  v = fmaxf(v, dpp<kDppBcast31, 0xc>(-__builtin_huge_valf(), v));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Sum over the whole wave, returned as a wave-uniform value.
__device__ inline float wave_sum_u(float v) {
  v += dpp<kDppXor1>(v, v);
  v += dpp<kDppXor2>(v, v);
  v += dpp<kDppHalfMirror>(v, v);
  v += dpp<kDppMirror>(v, v);
  v += dpp<kDppBcast15, 0xa>(0.f, v);
  v += dpp<kDppBcast31, 0xc>(0.f, v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Wave-wide reductions over all 64 lanes.
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Max over aligned groups of `width` lanes (width a power of two <= 64).
__device__ inline float group_max(float v, int width) {
  for (int off = width >> 1; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// Order-preserving map float -> uint32 (larger float, larger key); -0 == +0.
__device__ inline uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------------------
// Persistent work lists. A kernel's work is a list of chunks, sequence by
// sequence; chunk counts depend on device-side lengths, so each workgroup
// builds the exclusive prefix s_base[0..batch] of per-sequence chunk counts
// in LDS (wave 0, 64 sequences per step) and then walks the list with a
// grid stride. count(b) must be >= 1.
template <class CountFn>
__device__ inline void build_chunk_prefix(int batch, int* s_base, CountFn count) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    int carry = 0;
    for (int b0 = 0; b0 < batch; b0 += kWave) {
      const int b = b0 + lane;
      int c = (b < batch) ? count(b) : 0;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int t = __shfl_up(c, off, kWave);
        if (lane >= off) c += t;
      }
      if (b < batch) s_base[b + 1] = carry + c;
      carry += __shfl(c, kWave - 1, kWave);
    }
    if (lane == 0) s_base[0] = 0;
  }
  __syncthreads();
}

// Largest b with s_base[b] <= w (s_base strictly increasing, s_base[0] = 0).
__device__ inline int find_sequence(const int* s_base, int batch, int w) {
  int lo = 0, hi = batch;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_base[mid] <= w) lo = mid; else hi = mid;
  }
  return lo;
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

}  // namespace kvlr
