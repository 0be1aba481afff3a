// Embedding amplification by layer normalisation (section 3.2.4 of the deep-notes page on
// "Scaling Embeddings Outperforms Scaling Experts in Language Models": a LayerNorm on the
// layer output before it joins the residual stream; the pages give no formula, the usual
// one is taken):
//   out[r, :] = (e_r - mean_r) / sqrt(var_r + eps) * weight + bias
// over the D values of row r, var the biased variance, from the unrounded fp32 rows e that
// the projection left in the workspace. Rows whose token is outside [0, V0) (bad ids,
// unused decode slots) are written as zeros, like the plain layer's.
//
// One wave per row (4 rows per 256-thread block): each lane loads its NV 16-byte vectors of
// the row at once (consecutive lanes on consecutive vectors), together with its parameters
// and the row's token; the two reductions (the mean, then the centred squares, so no
// cancellation) stay inside the wave in a fixed order, and the row is written once, rounded
// once. NV is picked per D from a few sizes so the row sits
// in registers. Both streams are touched once, so loads and stores are non-temporal (about
// 2% faster on the 64K-token batch). HBM-bound: 4D bytes read and D * esz written per row.
#include <algorithm>

#include "bf16.h"
#include "kernels.h"

namespace ngram {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / 64;

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Sum over the wave in a fixed order (butterfly): every lane ends with the same total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <typename T>
__device__ __forceinline__ void store4(T* p, int c4, f32x4_t y);
template <>
__device__ __forceinline__ void store4<float>(float* p, int c4, f32x4_t y) {
  __builtin_nontemporal_store(y, reinterpret_cast<f32x4_t*>(p) + c4);
}
template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t* p, int c4, f32x4_t y) {
  u32x2_t h;
  h.x = f32_to_bf16_rne(y.x) | (f32_to_bf16_rne(y.y) << 16);
  h.y = f32_to_bf16_rne(y.z) | (f32_to_bf16_rne(y.w) << 16);
  __builtin_nontemporal_store(h, reinterpret_cast<u32x2_t*>(p) + c4);
}

// 4 consecutive parameters (weight or bias) as loaded (bf16 pairs or fp32), and as fp32
// when used (`fill` when the pointer is null)
template <typename T> struct Param4;
template <> struct Param4<float> {
  typedef f32x4_t raw;
  static __device__ __forceinline__ raw load(const float* p, int c4) {
    return p ? reinterpret_cast<const f32x4_t*>(p)[c4] : f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  static __device__ __forceinline__ f32x4_t get(const float* p, raw v, float fill) {
    return p ? v : f32x4_t{fill, fill, fill, fill};
  }
};
template <> struct Param4<uint16_t> {
  typedef u32x2_t raw;
  static __device__ __forceinline__ raw load(const uint16_t* p, int c4) {
    return p ? reinterpret_cast<const u32x2_t*>(p)[c4] : u32x2_t{0u, 0u};
  }
  static __device__ __forceinline__ f32x4_t get(const uint16_t* p, raw h, float fill) {
    if (!p) return f32x4_t{fill, fill, fill, fill};
    return f32x4_t{bf16_to_f32(h.x & 0xffffu), bf16_to_f32(h.x >> 16),
                   bf16_to_f32(h.y & 0xffffu), bf16_to_f32(h.y >> 16)};
  }
};

template <typename T, int NV>
__global__ __launch_bounds__(kThreads) void layernorm_rows_kernel(
    const float* __restrict__ pre, const int32_t* __restrict__ tok, int32_t V0,
    const T* __restrict__ weight, const T* __restrict__ bias, float eps, int32_t D,
    int64_t nrows, T* __restrict__ out, RowMap map) {
  const int64_t r = int64_t(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= nrows) return;                        // whole waves leave; no barrier follows
  const int D4 = D / 4;
  // The token, the row and the parameters are all requested before any is used: one memory
  // round trip per wave (the row's address does not depend on its token; rows that turn out
  // skipped or invalid only waste their loads). 234 -> 205 us on the 64K-token batch. The
  // parameters are held early only while they take at most 48 registers (bf16 rows up to
  // D = 3072, fp32 up to 1024); wider rows load them when used, to keep occupancy.
  constexpr bool kEarly = NV * int(sizeof(typename Param4<T>::raw)) / 2 <= 48;
  const int32_t tk = tok[r];
  const f32x4_t* src = reinterpret_cast<const f32x4_t*>(pre + r * D);
  f32x4_t v[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int c4 = lane + k * 64;
    v[k] = c4 < D4 ? __builtin_nontemporal_load(src + c4) : f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  typename Param4<T>::raw wr[kEarly ? NV : 1], br[kEarly ? NV : 1];
  if constexpr (kEarly) {
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int c4 = lane + k * 64;
      wr[k] = c4 < D4 ? Param4<T>::load(weight, c4) : typename Param4<T>::raw{};
      br[k] = c4 < D4 ? Param4<T>::load(bias, c4) : typename Param4<T>::raw{};
    }
  }
  if (tk == kSkipRow) return;                    // a row that is not written
  const int64_t orow = map.group ? (r / map.group) * map.stride + map.off + r % map.group : r;
  T* o = out + orow * D;
  if (uint32_t(tk) >= uint32_t(V0)) {            // the whole wave takes this branch
    for (int c4 = lane; c4 < D4; c4 += 64) store4<T>(o, c4, f32x4_t{0.f, 0.f, 0.f, 0.f});
    return;
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < NV; ++k) s += (v[k].x + v[k].y) + (v[k].z + v[k].w);
  const float mean = wave_sum(s) / float(D);
  float q = 0.f;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    if (lane + k * 64 < D4) {
      const f32x4_t c = v[k] - mean;
      q += (c.x * c.x + c.y * c.y) + (c.z * c.z + c.w * c.w);
    }
  }
  const float var = wave_sum(q) / float(D);
  const float rstd = 1.0f / sqrtf(var + eps);
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int c4 = lane + k * 64;
    if (c4 < D4) {
      const typename Param4<T>::raw wk = kEarly ? wr[k] : Param4<T>::load(weight, c4);
      const typename Param4<T>::raw bk = kEarly ? br[k] : Param4<T>::load(bias, c4);
      const f32x4_t y = (v[k] - mean) * rstd * Param4<T>::get(weight, wk, 1.f) +
                        Param4<T>::get(bias, bk, 0.f);
      store4<T>(o, c4, y);
    }
  }
}

template <typename T, int NV>
hipError_t launch_rows(const LayerDesc& L, const float* pre, const int32_t* tok,
                       const void* weight, const void* bias, int64_t nrows, void* out,
                       const RowMap& map, hipStream_t st) {
  const int64_t chunk = int64_t(1) << 30;        // rows per launch keeps the grid in range
  if (map.group != 0 && nrows > chunk) return hipErrorInvalidValue;
  for (int64_t r0 = 0; r0 < nrows; r0 += chunk) {
    const int64_t n = std::min(chunk, nrows - r0);
    hipLaunchKernelGGL((layernorm_rows_kernel<T, NV>),
                       dim3(unsigned((n + kRowsPerBlock - 1) / kRowsPerBlock)), dim3(kThreads),
                       0, st, pre + r0 * L.D, tok + r0, L.V0, static_cast<const T*>(weight),
                       static_cast<const T*>(bias), L.ln_eps, L.D, n,
                       static_cast<T*>(out) + r0 * L.D, map);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename T>
hipError_t launch_typed(const LayerDesc& L, const float* pre, const int32_t* tok,
                        const void* weight, const void* bias, int64_t nrows, void* out,
                        const RowMap& map, hipStream_t st) {
  // 16-byte vectors per lane: the smallest listed size that holds D / 256 of them
  const int need = (L.D / 4 + 63) / 64;
  if (need <= 2) return launch_rows<T, 2>(L, pre, tok, weight, bias, nrows, out, map, st);
  if (need <= 4) return launch_rows<T, 4>(L, pre, tok, weight, bias, nrows, out, map, st);
  if (need <= 8) return launch_rows<T, 8>(L, pre, tok, weight, bias, nrows, out, map, st);
  if (need <= 12) return launch_rows<T, 12>(L, pre, tok, weight, bias, nrows, out, map, st);
  if (need <= 16) return launch_rows<T, 16>(L, pre, tok, weight, bias, nrows, out, map, st);
  if (need <= 24) return launch_rows<T, 24>(L, pre, tok, weight, bias, nrows, out, map, st);
  return launch_rows<T, kMaxNormD / 256>(L, pre, tok, weight, bias, nrows, out, map, st);
}

}  // namespace

hipError_t launch_layernorm(const LayerDesc& L, const float* pre, const int32_t* tok,
                            const void* weight, const void* bias, int64_t nrows, void* out,
                            const RowMap& map, hipStream_t st) {
  if (nrows <= 0) return hipSuccess;
  if (L.dtype == NGRAM_F32)
    return launch_typed<float>(L, pre, tok, weight, bias, nrows, out, map, st);
  return launch_typed<uint16_t>(L, pre, tok, weight, bias, nrows, out, map, st);
}

}  // namespace ngram
