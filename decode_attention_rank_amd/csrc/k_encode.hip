// Append-side encode of new keys and values into the paged latent cache.
//
// BasisKV: Value Latents for Communication and Key Routing, English abstract:
// keys and values are compressed on write by low-rank projections; the value
// latent is stored, and what it cannot predict of the key is kept as a
// key-specific residual latent next to the original key.
//   v = RNE(V A_v)
//   routed: c = RNE((K - v W_pred) A_k), original key copied to its page
//   dense:  k = RNE(K A_k)
// These are true dense contractions and run on the matrix cores
// (bf16: v_mfma_f32_16x16x32_bf16; f32: v_mfma_f32_16x16x4_f32) with float32
// accumulation. The routed residual is evaluated as
//   c = K A_k + v (-(W_pred A_k)),
// an exact reassociation of the definition: the r_v x r_k matrix
// W_pred A_k is formed once per workgroup on the matrix cores, negated and,
// for bf16, split into a high and a low bf16 part so the product with the
// stored (bf16) latent v keeps about 16 significant bits of the matrix.
//
// Work split: grid (token-tile groups, KV head). A workgroup stages the
// factor fragments of its head in LDS once, then loops over 64-token tiles,
// 16 tokens per wave: the wave loads its tokens' rows straight into MFMA
// A-operand registers, multiplies, rounds into a per-wave LDS tile and writes
// each token's 16-byte chunks to its page slot.

#include "kvlr_device.h"
#include "kvlr_internal.h"

namespace kvlr {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

template <class S>
struct Mma;

template <>
struct Mma<BF16> {
  static constexpr int KSTEP = 32;  // k per instruction
  static constexpr int KPL = 8;     // k elements per lane
  using E = uint16_t;
  using frag_t = bf16x8;
  __device__ static f32x4 mma(frag_t a, frag_t b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static frag_t lds(const E* p) {
    return __builtin_bit_cast(frag_t, *reinterpret_cast<const uint4*>(p));
  }
  __device__ static frag_t gmem(const uint8_t* p) { return __builtin_bit_cast(frag_t, load16(p)); }
  __device__ static frag_t zero() { return __builtin_bit_cast(frag_t, make_uint4(0, 0, 0, 0)); }
  __device__ static E store(float f) { return static_cast<E>(f32_to_bf16_rne(f)); }
  __device__ static float value(E e) { return __uint_as_float(static_cast<uint32_t>(e) << 16); }
};

template <>
struct Mma<F32> {
  static constexpr int KSTEP = 4;
  static constexpr int KPL = 1;
  using E = float;
  using frag_t = float;
  __device__ static f32x4 mma(frag_t a, frag_t b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __device__ static frag_t lds(const E* p) { return *p; }
  __device__ static frag_t gmem(const uint8_t* p) { return *reinterpret_cast<const float*>(p); }
  __device__ static frag_t zero() { return 0.f; }
  __device__ static E store(float f) { return f; }
  __device__ static float value(E e) { return e; }
};

template <class S, int D, int RV, int RK, bool ROUTED>
struct EncSmem {
  using MM = Mma<S>;
  using E = typename MM::E;
  static constexpr int KSTEP = MM::KSTEP, KPL = MM::KPL, CH = S::CH;
  static constexpr int KSD = D / KSTEP;                    // k-steps over head_dim
  static constexpr int KSV = (RV + KSTEP - 1) / KSTEP;     // k-steps over rank_v (zero padded)
  // B-operand fragments: [k-step][n-tile][lane][KPL]
  alignas(16) E av[KSD][RV / 16][kWave][KPL];
  alignas(16) E ak[KSD][RK / 16][kWave][KPL];
  alignas(16) E mhi[ROUTED ? KSV : 1][RK / 16][kWave][KPL];
  alignas(16) E mlo[(ROUTED && KPL > 1) ? KSV : 1][RK / 16][kWave][KPL];
  float mstage[ROUTED ? RV : 1][RK + 1];
  // per-wave row-major tiles of the rounded latents (16 tokens)
  alignas(16) E vt[kWaves][16][RV + CH];
  alignas(16) E ct[kWaves][16][RK + CH];
};

__device__ inline void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

template <class S, int D, int RV, int RK, bool ROUTED>
__global__ __launch_bounds__(kThreads) void encode_kernel(
    const uint8_t* __restrict__ A_v, const uint8_t* __restrict__ A_k,
    const uint8_t* __restrict__ W_pred, const uint8_t* __restrict__ k_new,
    const uint8_t* __restrict__ v_new, const int32_t* __restrict__ cu_new,
    const int32_t* __restrict__ lens_before, const int32_t* __restrict__ page_table,
    uint8_t* __restrict__ v_lat, uint8_t* __restrict__ k_lat, uint8_t* __restrict__ k_exact,
    int Hkv, int P, int log2P, int max_pages, int batch, int total_new) {
  using MM = Mma<S>;
  using SM = EncSmem<S, D, RV, RK, ROUTED>;
  using E = typename MM::E;
  using frag_t = typename MM::frag_t;
  constexpr int KSTEP = MM::KSTEP, KPL = MM::KPL, CH = S::CH, EB = S::ELEM_BYTES;
  constexpr int KSD = SM::KSD, KSV = SM::KSV;
  constexpr int NTV = RV / 16, NTK = RK / 16;
  constexpr int CV = RV / CH, CK = RK / CH, CD = D / CH;
  __shared__ SM sm;

  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid & (kWave - 1);
  const E* Av = reinterpret_cast<const E*>(A_v) + static_cast<size_t>(g) * D * RV;
  const E* Ak = reinterpret_cast<const E*>(A_k) + static_cast<size_t>(g) * D * RK;

  // ---- stage B fragments: element (k, n) with k = ks*KSTEP + KPL*(l/16) + e, n = nt*16 + l%16
  for (int idx = tid; idx < KSD * NTV * kWave * KPL; idx += kThreads) {
    const int e = idx % KPL, l = (idx / KPL) % kWave, nt = (idx / (KPL * kWave)) % NTV;
    const int ks = idx / (KPL * kWave * NTV);
    const int k = ks * KSTEP + KPL * (l >> 4) + e, n = nt * 16 + (l & 15);
    sm.av[ks][nt][l][e] = Av[k * RV + n];
  }
  for (int idx = tid; idx < KSD * NTK * kWave * KPL; idx += kThreads) {
    const int e = idx % KPL, l = (idx / KPL) % kWave, nt = (idx / (KPL * kWave)) % NTK;
    const int ks = idx / (KPL * kWave * NTK);
    const int k = ks * KSTEP + KPL * (l >> 4) + e, n = nt * 16 + (l & 15);
    sm.ak[ks][nt][l][e] = Ak[k * RK + n];
  }
  __syncthreads();

  if constexpr (ROUTED) {
    // M = W_pred A_k  [RV x RK], one 16x16 tile per wave at a time
    const uint8_t* Wg = W_pred + static_cast<size_t>(g) * RV * D * EB;
    for (int ti = wave; ti < NTV * NTK; ti += kWaves) {
      const int mt = ti / NTK, nt = ti - mt * NTK;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const int row = mt * 16 + (lane & 15);
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks) {
        const frag_t a = MM::gmem(Wg + (static_cast<size_t>(row) * D + ks * KSTEP + KPL * (lane >> 4)) * EB);
        acc = MM::mma(a, MM::lds(&sm.ak[ks][nt][lane][0]), acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.mstage[mt * 16 + 4 * (lane >> 4) + i][nt * 16 + (lane & 15)] = acc[i];
    }
    __syncthreads();
    for (int idx = tid; idx < KSV * NTK * kWave * KPL; idx += kThreads) {
      const int e = idx % KPL, l = (idx / KPL) % kWave, nt = (idx / (KPL * kWave)) % NTK;
      const int ks = idx / (KPL * kWave * NTK);
      const int k = ks * KSTEP + KPL * (l >> 4) + e, n = nt * 16 + (l & 15);
      const float mv = (k < RV) ? -sm.mstage[k][n] : 0.f;
      const E hi = MM::store(mv);
      sm.mhi[ks][nt][l][e] = hi;
      if constexpr (KPL > 1) sm.mlo[ks][nt][l][e] = MM::store(mv - MM::value(hi));
    }
    __syncthreads();
  }

  const int ntiles = (total_new + 63) / 64;
  const int r = lane & 15;        // A-operand row (token) of this lane
  const int kq = lane >> 4;       // A-operand k group of this lane
  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int i = tile * 64 + wave * 16 + r;
    const bool valid = i < total_new;
    size_t slot_off = 0, phys = 0;
    if (valid) {
      int lo = 0, hi = batch;  // largest b with cu_new[b] <= i
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cu_new[mid] <= i) lo = mid; else hi = mid;
      }
      const int pos = lens_before[lo] + (i - cu_new[lo]);
      phys = static_cast<size_t>(page_table[static_cast<size_t>(lo) * max_pages + (pos >> log2P)]);
      slot_off = static_cast<size_t>(pos & (P - 1)) * 16;
    }
    const size_t row_off = (static_cast<size_t>(valid ? i : 0) * Hkv + g) * D * EB;

    // ---- v = V A_v
    f32x4 vacc[NTV];
#pragma unroll
    for (int nt = 0; nt < NTV; ++nt) vacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) {
      const frag_t a = valid ? MM::gmem(v_new + row_off + (ks * KSTEP + KPL * kq) * EB) : MM::zero();
#pragma unroll
      for (int nt = 0; nt < NTV; ++nt) vacc[nt] = MM::mma(a, MM::lds(&sm.av[ks][nt][lane][0]), vacc[nt]);
    }
#pragma unroll
    for (int nt = 0; nt < NTV; ++nt)
#pragma unroll
      for (int j = 0; j < 4; ++j) sm.vt[wave][4 * kq + j][nt * 16 + r] = MM::store(vacc[nt][j]);
    wave_lds_sync();
    if (valid) {
      uint8_t* dst = v_lat + (phys * Hkv + g) * CV * P * 16 + slot_off;
      for (int c = kq; c < CV; c += 4)
        store16(dst + static_cast<size_t>(c) * P * 16, *reinterpret_cast<const uint4*>(&sm.vt[wave][r][c * CH]));
    }

    // ---- residual latent (routed) or key latent (dense)
    f32x4 cacc[NTK];
#pragma unroll
    for (int nt = 0; nt < NTK; ++nt) cacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) {
      const frag_t a = valid ? MM::gmem(k_new + row_off + (ks * KSTEP + KPL * kq) * EB) : MM::zero();
#pragma unroll
      for (int nt = 0; nt < NTK; ++nt) cacc[nt] = MM::mma(a, MM::lds(&sm.ak[ks][nt][lane][0]), cacc[nt]);
    }
    if constexpr (ROUTED) {
#pragma unroll
      for (int ks = 0; ks < KSV; ++ks) {
        const int k = ks * KSTEP + KPL * kq;
        const frag_t a = (k < RV) ? MM::lds(&sm.vt[wave][r][k]) : MM::zero();
#pragma unroll
        for (int nt = 0; nt < NTK; ++nt) {
          cacc[nt] = MM::mma(a, MM::lds(&sm.mhi[ks][nt][lane][0]), cacc[nt]);
          if constexpr (KPL > 1) cacc[nt] = MM::mma(a, MM::lds(&sm.mlo[ks][nt][lane][0]), cacc[nt]);
        }
      }
    }
#pragma unroll
    for (int nt = 0; nt < NTK; ++nt)
#pragma unroll
      for (int j = 0; j < 4; ++j) sm.ct[wave][4 * kq + j][nt * 16 + r] = MM::store(cacc[nt][j]);
    wave_lds_sync();
    if (valid) {
      uint8_t* dst = k_lat + (phys * Hkv + g) * CK * P * 16 + slot_off;
      for (int c = kq; c < CK; c += 4)
        store16(dst + static_cast<size_t>(c) * P * 16, *reinterpret_cast<const uint4*>(&sm.ct[wave][r][c * CH]));
      if constexpr (ROUTED) {
        uint8_t* kd = k_exact + (phys * Hkv + g) * CD * P * 16 + slot_off;
        for (int c = kq; c < CD; c += 4)
          store16(kd + static_cast<size_t>(c) * P * 16, load16(k_new + row_off + c * 16));
      }
    }
    wave_lds_sync();
  }
}

template <class S, int D, int RV, int RK, bool ROUTED>
hipError_t launch_t(const EncodeArgs& a, hipStream_t s) {
  const int log2P = __builtin_ctz(static_cast<unsigned>(a.dm.P));
  const int ntiles = (a.total_new + 63) / 64;
  int per_head = (2048 + a.dm.Hkv - 1) / a.dm.Hkv;
  if (per_head > ntiles) per_head = ntiles;
  dim3 grid(per_head, a.dm.Hkv);
  hipLaunchKernelGGL((encode_kernel<S, D, RV, RK, ROUTED>), grid, dim3(kThreads), 0, s,
                     static_cast<const uint8_t*>(a.A_v), static_cast<const uint8_t*>(a.A_k),
                     static_cast<const uint8_t*>(a.W_pred), static_cast<const uint8_t*>(a.k_new),
                     static_cast<const uint8_t*>(a.v_new), a.cu_new, a.lens_before, a.page_table,
                     static_cast<uint8_t*>(a.v_lat), static_cast<uint8_t*>(a.k_lat),
                     static_cast<uint8_t*>(a.k_exact), a.dm.Hkv, a.dm.P, log2P, a.max_pages,
                     a.batch, a.total_new);
  return hipGetLastError();
}

template <class S, int D, int RV, int RK>
hipError_t by_mode(const EncodeArgs& a, hipStream_t s) {
  return a.dm.exact ? launch_t<S, D, RV, RK, true>(a, s) : launch_t<S, D, RV, RK, false>(a, s);
}

template <class S, int D, int RV>
hipError_t by_rk(const EncodeArgs& a, hipStream_t s) {
  switch (a.dm.RK) {
    case 16: return by_mode<S, D, RV, 16>(a, s);
    case 32: return by_mode<S, D, RV, 32>(a, s);
    case 64: return by_mode<S, D, RV, 64>(a, s);
  }
  return hipErrorInvalidValue;
}

template <class S, int D>
hipError_t by_rv(const EncodeArgs& a, hipStream_t s) {
  switch (a.dm.RV) {
    case 16: return by_rk<S, D, 16>(a, s);
    case 32: return by_rk<S, D, 32>(a, s);
    case 64: return by_rk<S, D, 64>(a, s);
  }
  return hipErrorInvalidValue;
}

template <class S>
hipError_t by_d(const EncodeArgs& a, hipStream_t s) {
  switch (a.dm.D) {
    case 64: return by_rv<S, 64>(a, s);
    case 128: return by_rv<S, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_encode(const EncodeArgs& a, hipStream_t s) {
  if (a.total_new == 0 || a.batch == 0) return hipSuccess;
  if (a.dm.dtype == 0) return by_d<BF16>(a, s);
  return by_d<F32>(a, s);
}

}  // namespace kvlr
